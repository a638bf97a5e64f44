// Stream probe (measurement only) — host interface.
#pragma once

#include "common.h"

namespace ql {

// Tiles of rd KB read and wr KB written; (rd, wr) in {(1, 0), (4, 1), (1, 4)};
// depth tiles per wave and pass (1, 2, 4 or 8); blocks workgroups of 256
// threads, or 0 for min(ceil(ntiles / 8), 8192).
hipError_t launch_stream_probe(int rd, int wr, int depth, int blocks, const void *src, void *dst, int64_t ntiles,
                               hipStream_t st);

}  // namespace ql
