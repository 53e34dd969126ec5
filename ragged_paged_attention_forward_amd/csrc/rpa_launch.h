// Interface between the host library (rpa_api.cpp) and the kernel dispatch
// (rpa_dispatch.cpp, which calls the per-head-size rpa_kernels_d*.hip units).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "rpa.h"

namespace rpa {

struct LaunchArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* page_table;
  void* out;
  const rpa_work_item* groups;  // device
  float* partial_o;             // device [slots][16][D]
  float* partial_lse;           // device [slots][16]
  int32_t* merge_tickets;       // device [groups], zero between calls
  int32_t fused_merge;          // 1: decode kernel merges split groups itself
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_pages;
  int32_t window;
  float scale_log2;
  int32_t decode_waves;  // waves per decode workgroup: 4 or 8
  int32_t kv_fp8;        // 1: k / v hold OCP FP8 E4M3 bytes with per-KV-head scales
  const float* k_scales; // device [Hkv] (fp8 only)
  const float* v_scales; // device [Hkv] (fp8 only)
  const void* k_new;     // appending calls: new K rows [T, Hkv, D] bf16 (else null)
  const void* v_new;     // appending calls: new V rows (else null)
  int32_t prefill_writes;  // appending calls: 1 the prefill kernel writes its items' new rows
  void* stream;
};

// Rows (tokens x grouped heads) per prefill workgroup for a head size, 0 if none.
int prefill_rows_for(int head_dim);
// Prefill workgroups one compute unit holds at once for a head size.
int prefill_wgs_per_cu_for(int head_dim);
// bf16 tiles the prefill kernel's E4M3 form converts into per workgroup: 2
// (the next tile is converted while the current one is used) or 1 (after
// its products, behind a second barrier).
int prefill_fp8_tiles_for(int head_dim);
bool head_dim_supported(int head_dim);

// alone: the call has no decode items (the prefill launch has the compute
// units to itself), which picks the head size's prefill-only tile shape for
// a bf16 launch.
hipError_t launch_prefill(const LaunchArgs& a, const rpa_work_item* items, int n_items, bool alone);
// Whether a bf16 prefill launch (shape chosen by `alone`) can take an
// appending call's new rows itself: its K/V loads go in runs of keys that
// lie in one page (a tile, or a wave's rows of one), and every sequence's
// first new position (a multiple of new_align) must start a run, so that no
// run holds both pool rows and new rows; with a page id per lane, always.
bool prefill_takes_new_rows(const LaunchArgs& a, bool alone, int new_align);
// rows: 16 for the one-block decode kernel, 32 for the two-block one.
hipError_t launch_decode(const LaunchArgs& a, const rpa_work_item* items, int n_items, int rows);
// Merges split groups a.groups[0 .. n_groups) (max_rows: the most rows of a
// split among them), several workgroups per group.
hipError_t launch_merge(const LaunchArgs& a, int n_groups, int max_rows);
// Copies the step's new K/V rows (k_new / v_new, [T, Hkv, D]) into their page
// slots of k_dst / v_dst, one workgroup per work item.
hipError_t launch_append(const LaunchArgs& a, const rpa_work_item* items, int n_items, const void* k_new,
                         const void* v_new, void* k_dst, void* v_dst);
// fp8 calls: converts the staged pages (stage: 3 ints per page, device) of
// the fp8 pools a.k / a.v (page ids from a.page_table) to bf16 pages of
// k_dst / v_dst, scaled by a.k_scales / a.v_scales.
hipError_t launch_stage(const LaunchArgs& a, const int32_t* stage, int n_pages, void* k_dst, void* v_dst);

}  // namespace rpa
