// Host-side ragged metadata builder: turns per-sequence query/KV lengths into
// the work lists the attention kernels consume.  Pure C++ (no HIP), so it is
// also exercised on machines without a GPU through rpa_plan().
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "rpa.h"

namespace rpa {

struct PlanParams {
  int num_q_heads = 0;
  int num_kv_heads = 0;
  int head_dim = 0;
  int page_size = 0;
  int max_num_seqs = 0;
  int max_pages_per_seq = 0;
  int64_t max_q_tokens = 0;
  int prefill_rows = 128;      // query rows (tokens x grouped heads) per prefill tile
  int prefill_wgs_per_cu = 1;  // prefill workgroups one compute unit holds at once
  int decode_max_rows = 0;     // most rows of one decode item, 0 = the tuning table
                               // (decode_rows_limit); items of up to 16 rows run the one-block
                               // decode kernel, of 17..32 rows the two-block one (head sizes
                               // up to 256; 512 stops at 16)
  int decode_wave_keys = 32;   // keys one decode wave takes per step
  int decode_waves = 4;        // waves of one decode workgroup
  int64_t decode_split_keys = 0;  // 0: automatic
  int64_t prefill_split_keys = 0; // 0: automatic, < 0: never, > 0: fixed
  int path_mode = 0;           // 0 auto, 1 all prefill kernel, 2 decode where it fits,
                               // 3 every token through decode items (long sequences in chunks)
  int num_cus = 256;           // compute units to fill
  int xcd_groups = 8;          // prefill order: workgroups b, b+X, b+2X, ... share a
                               // chiplet (and its L2); <= 1 keeps the plain order
  int xcd_run = 4;             // consecutive items dealt to one chiplet at a time
  bool kv8 = false;            // an fp8 (E4M3) cache
  bool stage_prefill = false;  // fp8 calls (RPA_OPT_FP8_STAGE): the pages of sequences with
                               // prefill items are staged into a bf16 pool that the prefill
                               // kernel reads
};

struct Plan {
  std::vector<rpa_work_item> prefill;  // launch order
  std::vector<rpa_work_item> decode;   // launch order, items of up to 16 rows (kind 1)
  std::vector<rpa_work_item> decode2;  // launch order, items of 17..32 rows (kind 2)
  std::vector<rpa_work_item> groups;   // one entry per split group (its split 0): prefill groups first
  int32_t prefill_groups = 0;          // groups[0 .. prefill_groups) are prefill split groups
  int num_partials = 0;                // 16-row partial-result slots (a prefill split takes rows/16,
                                       // a two-block decode split 2)
  int prefill_split_keys = 0;          // keys per prefill split chosen (0: none split)
  int decode_split_keys = 0;
  int64_t visible_pairs = 0;
  int64_t total_q = 0;
  int32_t append_items = 0;            // items whose new rows the append kernel writes (the others
                                       // write their own in the decode or prefill kernel)
  int32_t prefill_writer_items = 0;    // prefill items that write their query tokens' rows (bf16):
                                       // the append kernel takes them when the prefill kernel cannot
  int32_t new_align = 0;               // largest power of two (up to 2^30) dividing the first new
                                       // position of every sequence served by prefill items
  // Staging (stage_prefill): three ints per staged page (sequence, page of
  // the sequence, page of the bf16 pool), and the bf16 pool's page table
  // [num_seqs * max_pages_per_seq] (rows of staged sequences; 0 elsewhere).
  std::vector<int32_t> stage;
  std::vector<int32_t> stage_table;
  int32_t stage_pages = 0;
};

// Checks the metadata of one call.  Returns RPA_OK or RPA_ERR_INVALID_ARG with *err set.
int validate_metadata(const PlanParams& p, const int32_t* cu_q_lens, const int32_t* kv_lens,
                      int32_t num_seqs, int32_t window, std::string* err);

// Builds the work lists (metadata must have passed validate_metadata).
void build_plan(const PlanParams& p, const int32_t* cu_q_lens, const int32_t* kv_lens,
                int32_t num_seqs, int32_t window, Plan* out);

// The tuning table's decode regime: the most rows (query tokens x grouped
// heads) of a sequence that the decode kernels take; sequences with more
// rows go to the prefill kernel.  Measured on MI355X (128 sequences, keys
// U[64, 1024], 32-row steps: G = 32 x 1 token, G = 8 x 4 tokens):
//   bf16 cache: the prefill kernel (its few-row items cut into short key
//     pieces) is as fast as the two-block decode kernel at head sizes 64
//     and 128 and 22 % faster at 256 (where the two-block kernel holds one
//     wave per SIMD) -> 16 rows;
//   fp8 cache: the prefill kernel first stages the sequences' pages to bf16,
//     so the two-block decode kernel, which converts in registers, is 1.5-2x
//     faster (d 64: 14.3 against 24.6 us; d 128: 17.6 against 33.9; d 256:
//     38.8 against 56.5) -> 32 rows for head sizes up to 256.
// Head size 512 has no two-block kernel: 16 rows.  A non-zero
// RPA_OPT_DECODE_MAX_ROWS replaces the table's value (within that cap).
inline int decode_rows_limit(const PlanParams& p) {
  const int cap = p.head_dim <= 256 ? 32 : 16;
  const int want = p.decode_max_rows > 0 ? p.decode_max_rows : (p.kv8 ? 32 : 16);
  return want < cap ? want : cap;
}

// Number of visible keys of query position `pos` (keys 0..pos, clipped by the window).
inline int64_t visible_keys(int64_t pos, int32_t window) {
  if (window > 0 && pos + 1 > window) return window;
  return pos + 1;
}

}  // namespace rpa
