// Host-side dispatch from the C ABI's launch arguments to the per-head-size
// kernel translation units.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rpa.h"
#include "rpa_kargs.h"
#include "rpa_launch.h"

namespace rpa {

hipError_t launch_prefill_d64(const KernelArgs& a, int n, bool kv8, hipStream_t s);
hipError_t launch_prefill_alone_d64(const KernelArgs& a, int n, hipStream_t s);
hipError_t launch_decode_d64(const KernelArgs& a, int n, int waves, bool kv8, int rows, hipStream_t s);
hipError_t launch_merge_d64(const KernelArgs& a, int n, int rows, hipStream_t s);
hipError_t launch_append_d64(const KernelArgs& a, int n, const void* kn, const void* vn, void* kd, void* vd,
                              bool kv8, hipStream_t s);
hipError_t launch_stage_d64(const KernelArgs& a, const int32_t* st, int n, void* kd, void* vd, hipStream_t s);
int prefill_rows_d64();
int prefill_wgs_per_cu_d64();
int prefill_fp8_tiles_d64();
int prefill_run_keys_d64(const KernelArgs& a, bool alone);
hipError_t launch_prefill_d128(const KernelArgs& a, int n, bool kv8, hipStream_t s);
hipError_t launch_prefill_alone_d128(const KernelArgs& a, int n, hipStream_t s);
hipError_t launch_decode_d128(const KernelArgs& a, int n, int waves, bool kv8, int rows, hipStream_t s);
hipError_t launch_merge_d128(const KernelArgs& a, int n, int rows, hipStream_t s);
hipError_t launch_append_d128(const KernelArgs& a, int n, const void* kn, const void* vn, void* kd, void* vd,
                              bool kv8, hipStream_t s);
hipError_t launch_stage_d128(const KernelArgs& a, const int32_t* st, int n, void* kd, void* vd, hipStream_t s);
int prefill_rows_d128();
int prefill_wgs_per_cu_d128();
int prefill_fp8_tiles_d128();
int prefill_run_keys_d128(const KernelArgs& a, bool alone);
hipError_t launch_prefill_d256(const KernelArgs& a, int n, bool kv8, hipStream_t s);
hipError_t launch_prefill_alone_d256(const KernelArgs& a, int n, hipStream_t s);
hipError_t launch_decode_d256(const KernelArgs& a, int n, int waves, bool kv8, int rows, hipStream_t s);
hipError_t launch_merge_d256(const KernelArgs& a, int n, int rows, hipStream_t s);
hipError_t launch_append_d256(const KernelArgs& a, int n, const void* kn, const void* vn, void* kd, void* vd,
                              bool kv8, hipStream_t s);
hipError_t launch_stage_d256(const KernelArgs& a, const int32_t* st, int n, void* kd, void* vd, hipStream_t s);
int prefill_rows_d256();
int prefill_wgs_per_cu_d256();
int prefill_fp8_tiles_d256();
int prefill_run_keys_d256(const KernelArgs& a, bool alone);
hipError_t launch_prefill_d512(const KernelArgs& a, int n, bool kv8, hipStream_t s);
hipError_t launch_prefill_alone_d512(const KernelArgs& a, int n, hipStream_t s);
hipError_t launch_decode_d512(const KernelArgs& a, int n, int waves, bool kv8, int rows, hipStream_t s);
hipError_t launch_merge_d512(const KernelArgs& a, int n, int rows, hipStream_t s);
hipError_t launch_append_d512(const KernelArgs& a, int n, const void* kn, const void* vn, void* kd, void* vd,
                              bool kv8, hipStream_t s);
hipError_t launch_stage_d512(const KernelArgs& a, const int32_t* st, int n, void* kd, void* vd, hipStream_t s);
int prefill_rows_d512();
int prefill_wgs_per_cu_d512();
int prefill_fp8_tiles_d512();
int prefill_run_keys_d512(const KernelArgs& a, bool alone);

int prefill_rows_for(int head_dim) {
  switch (head_dim) {
    case 64: return prefill_rows_d64();
    case 128: return prefill_rows_d128();
    case 256: return prefill_rows_d256();
    case 512: return prefill_rows_d512();
    default: return 0;
  }
}

bool head_dim_supported(int head_dim) { return prefill_rows_for(head_dim) > 0; }

int prefill_fp8_tiles_for(int head_dim) {
  switch (head_dim) {
    case 64: return prefill_fp8_tiles_d64();
    case 128: return prefill_fp8_tiles_d128();
    case 256: return prefill_fp8_tiles_d256();
    case 512: return prefill_fp8_tiles_d512();
    default: return 1;
  }
}

int prefill_wgs_per_cu_for(int head_dim) {
  switch (head_dim) {
    case 64: return prefill_wgs_per_cu_d64();
    case 128: return prefill_wgs_per_cu_d128();
    case 256: return prefill_wgs_per_cu_d256();
    case 512: return prefill_wgs_per_cu_d512();
    default: return 1;
  }
}

static KernelArgs make_args(const LaunchArgs& l, const rpa_work_item* items) {
  KernelArgs a;
  a.q = static_cast<const uint16_t*>(l.q);
  a.k = static_cast<const uint16_t*>(l.k);
  a.v = static_cast<const uint16_t*>(l.v);
  a.page_table = l.page_table;
  a.out = static_cast<uint16_t*>(l.out);
  a.items = items;
  a.groups = l.groups;
  a.partial_o = l.partial_o;
  a.partial_lse = l.partial_lse;
  a.merge_tickets = l.merge_tickets;
  a.fused_merge = l.fused_merge;
  a.num_q_heads = l.num_q_heads;
  a.num_kv_heads = l.num_kv_heads;
  a.group = l.num_q_heads / l.num_kv_heads;
  a.page_size = l.page_size;
  a.max_pages = l.max_pages;
  a.window = l.window;
  a.scale_log2 = l.scale_log2;
  a.prefill_rows = prefill_rows_for(l.head_dim);
  a.k_scales = l.k_scales;
  a.v_scales = l.v_scales;
  a.k_new = static_cast<const uint16_t*>(l.k_new);
  a.v_new = static_cast<const uint16_t*>(l.v_new);
  a.prefill_writes = l.prefill_writes;
  return a;
}

bool prefill_takes_new_rows(const LaunchArgs& l, bool alone, int new_align) {
  const KernelArgs a = make_args(l, nullptr);
  int run = 0;
  switch (l.head_dim) {
    case 64: run = prefill_run_keys_d64(a, alone); break;
    case 128: run = prefill_run_keys_d128(a, alone); break;
    case 256: run = prefill_run_keys_d256(a, alone); break;
    case 512: run = prefill_run_keys_d512(a, alone); break;
    default: return false;
  }
  return run == 0 || new_align % run == 0;
}

hipError_t launch_prefill(const LaunchArgs& l, const rpa_work_item* items, int n_items, bool alone) {
  if (n_items <= 0) return hipSuccess;
  const KernelArgs a = make_args(l, items);
  hipStream_t s = static_cast<hipStream_t>(l.stream);
  const bool kv8 = l.kv_fp8 != 0;
  if (alone && !kv8) {
    switch (l.head_dim) {
      case 64: return launch_prefill_alone_d64(a, n_items, s);
      case 128: return launch_prefill_alone_d128(a, n_items, s);
      case 256: return launch_prefill_alone_d256(a, n_items, s);
      case 512: return launch_prefill_alone_d512(a, n_items, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (l.head_dim) {
    case 64: return launch_prefill_d64(a, n_items, kv8, s);
    case 128: return launch_prefill_d128(a, n_items, kv8, s);
    case 256: return launch_prefill_d256(a, n_items, kv8, s);
    case 512: return launch_prefill_d512(a, n_items, kv8, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const LaunchArgs& l, const rpa_work_item* items, int n_items, int rows) {
  if (n_items <= 0) return hipSuccess;
  const KernelArgs a = make_args(l, items);
  hipStream_t s = static_cast<hipStream_t>(l.stream);
  const int w = l.decode_waves;
  const bool kv8 = l.kv_fp8 != 0;
  switch (l.head_dim) {
    case 64: return launch_decode_d64(a, n_items, w, kv8, rows, s);
    case 128: return launch_decode_d128(a, n_items, w, kv8, rows, s);
    case 256: return launch_decode_d256(a, n_items, w, kv8, rows, s);
    case 512: return launch_decode_d512(a, n_items, w, kv8, rows, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_append(const LaunchArgs& l, const rpa_work_item* items, int n_items, const void* k_new,
                         const void* v_new, void* k_dst, void* v_dst) {
  if (n_items <= 0) return hipSuccess;
  const KernelArgs a = make_args(l, items);
  hipStream_t s = static_cast<hipStream_t>(l.stream);
  switch (l.head_dim) {
    case 64: return launch_append_d64(a, n_items, k_new, v_new, k_dst, v_dst, l.kv_fp8 != 0, s);
    case 128: return launch_append_d128(a, n_items, k_new, v_new, k_dst, v_dst, l.kv_fp8 != 0, s);
    case 256: return launch_append_d256(a, n_items, k_new, v_new, k_dst, v_dst, l.kv_fp8 != 0, s);
    case 512: return launch_append_d512(a, n_items, k_new, v_new, k_dst, v_dst, l.kv_fp8 != 0, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stage(const LaunchArgs& l, const int32_t* stage, int n_pages, void* k_dst, void* v_dst) {
  if (n_pages <= 0) return hipSuccess;
  const KernelArgs a = make_args(l, nullptr);
  hipStream_t s = static_cast<hipStream_t>(l.stream);
  switch (l.head_dim) {
    case 64: return launch_stage_d64(a, stage, n_pages, k_dst, v_dst, s);
    case 128: return launch_stage_d128(a, stage, n_pages, k_dst, v_dst, s);
    case 256: return launch_stage_d256(a, stage, n_pages, k_dst, v_dst, s);
    case 512: return launch_stage_d512(a, stage, n_pages, k_dst, v_dst, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_merge(const LaunchArgs& l, int n_groups, int max_rows) {
  if (n_groups <= 0) return hipSuccess;
  const KernelArgs a = make_args(l, nullptr);
  hipStream_t s = static_cast<hipStream_t>(l.stream);
  switch (l.head_dim) {
    case 64: return launch_merge_d64(a, n_groups, max_rows, s);
    case 128: return launch_merge_d128(a, n_groups, max_rows, s);
    case 256: return launch_merge_d256(a, n_groups, max_rows, s);
    case 512: return launch_merge_d512(a, n_groups, max_rows, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rpa
