// The library-held dgamma scratch of rmsnorm_bwd_noalloc (scratch.hip): its
// size and the host-side lookup of its device address. Plain types only.
#pragma once

#include <stddef.h>

namespace rmsn {

// Bytes of the scratch (one copy per GPU). The dgamma partials need at most
// 256 chunks x 32768 floats (rmsnorm_bwd_workspace_bytes; 512 chunks only
// for rows of at most 2048 elements), 32 MiB, so every supported shape fits.
constexpr size_t kScratchBytes = size_t{32} << 20;

// The device address of the current device's copy of the scratch (looked up
// once per device). Returns 0, or the HIP error code of a failed lookup.
int scratch_ptr(void** out);

}  // namespace rmsn
