// Launcher of the contraction probe (a measurement aid, not a step of the
// indexer): 128-dim fp8 dot products through one of three MFMA forms.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa_indexer.h"

namespace msa {

// out[tile, i, j] = q[tile, i, :] . k[tile, j, :] for 16 x 16 rows per tile,
// in the MFMA form `form` (MSA_PROBE_*).
hipError_t launch_contraction_probe(const uint8_t* q, const uint8_t* k, int64_t tiles, int form,
                                    float* out, hipStream_t stream);

}  // namespace msa
