// Kernels for head size 128 (one translation unit per head size, so each can
// be compiled with its own register-allocation options).
#include "rpa_device.h"

namespace rpa {
RPA_DEFINE_HEAD_DIM(128)
}  // namespace rpa
