// Internal interface between the no-allocation entry point (rpa_noalloc.hip,
// which owns the static scratch array) and the host library (rpa_api.cpp).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "rpa.h"

namespace rpa {

// Device address of the scratch array on `device` (the current device),
// or an error status.
typedef int (*ScratchResolver)(int device, void** ptr);

// rpa_forward with the work list and split partials in the scratch array
// (device memory of `scratch_bytes`, found through `resolve` once the host
// checks have passed), allocating nothing.
int forward_scratch(rpa_ctx* c, const void* q, const void* k_pages, const void* v_pages, const int32_t* page_table,
                    const int32_t* cu, const int32_t* kv, int32_t num_seqs, int32_t window, float scale, void* out,
                    void* stream, ScratchResolver resolve, size_t scratch_bytes);

}  // namespace rpa
