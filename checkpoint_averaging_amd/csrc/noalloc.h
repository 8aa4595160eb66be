// Internal interface of the allocation-free outer step's scratch (noalloc.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlk {

// The allocation-free outer step's scratch: a file-scope device array of
// kNoallocScratchBytes per device (noalloc.hip), which must hold a matrix's
// polar_workspace_bytes.  192 MiB holds the workspace of every weight matrix
// of DiffuRefill-1B but its embedding (at most 184 MiB, for the 5632 x 2048
// and 2048 x 5632 MLP matrices) and of Pythia-14M (at most 73.3 MiB).
constexpr int64_t kNoallocScratchBytes = int64_t(192) << 20;

// Device address of that array on `device`, which must be the calling
// thread's current device the first time it is asked for; looked up once
// per device with hipGetSymbolAddress and kept.
hipError_t noalloc_scratch(int device, void** addr);

}  // namespace dlk
