// Kernel argument block shared by the host dispatch and the device code.
#pragma once

#include <stdint.h>

#include "rpa.h"

namespace rpa {

struct KernelArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* page_table;
  uint16_t* out;
  const rpa_work_item* items;
  const rpa_work_item* groups;
  float* partial_o;      // [slot][16 rows][D]; a prefill split uses prefill_rows / 16 slots
  float* partial_lse;    // [slot][16 rows], base-2 log-sum-exp
  int32_t* merge_tickets;  // [group] splits finished so far (0 between calls)
  int32_t fused_merge;   // decode kernel: 1 the last split of a group merges it (no merge kernel)
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;         // G = Hq / Hkv
  int32_t page_size;
  int32_t max_pages;
  int32_t window;
  float scale_log2;      // scale * log2(e)
  int32_t prefill_rows;  // rows of a prefill tile (rows of a prefill split's partial block)
  const float* k_scales; // fp8 pools: K scale per KV head (else unused)
  const float* v_scales; // fp8 pools: V scale per KV head (else unused)
  const uint16_t* k_new; // appending calls: the step's new K rows [T, Hkv, D] bf16 (else null)
  const uint16_t* v_new; // appending calls: the step's new V rows (else null)
  int32_t prefill_writes; // appending calls: 1 the prefill kernel writes its items' new rows (the
                          // append kernel skips them)
};

}  // namespace rpa
