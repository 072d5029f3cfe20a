// Launcher of the streaming-read probe (a measurement aid, not a step of the
// indexer): a plain read of a buffer with no other work, so its rate is the
// streaming ceiling the scorer's rate is read against.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa_indexer.h"

namespace msa {

constexpr int64_t kProbeBlockBytes = 16384;  // one B128 block of index-K rows
constexpr int kProbeSinkWords = MSA_STREAM_PROBE_SINK_WORDS;

// Reads `blocks` contiguous 16 KiB blocks of src, blocks_per_wave (2, 4, 8
// or 16) consecutive ones per wave, or with MSA_STREAM_PROBE_PERSISTENT one
// contiguous run per wave of a grid of one wave per SIMD (anything else:
// hipErrorInvalidValue), and xors every dword of them into sink[0 ..
// kProbeSinkWords): wave w's share goes to word w % kProbeSinkWords, so that
// no single word takes every wave's atomic.
hipError_t launch_stream_read_probe(const uint8_t* src, int64_t blocks, int blocks_per_wave,
                                    uint32_t* sink, hipStream_t stream);

}  // namespace msa
