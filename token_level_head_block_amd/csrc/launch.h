// launch.h -- internal launchers of the libmhla kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace mhla {

struct Tuning {
    int summary_waves;   // waves splitting the tokens of one block in block_kv_summary (1, 2, 4)
    int apply_waves;     // waves splitting the tokens of one block in query_apply (1, 2, 4)
};

struct Launch {
    const void* q;
    const void* k;
    const void* v;
    const float* W;
    void* out;
    void* sz;      // summaries  [BH][M][D*D + D]   (compute type)
    void* st;      // mixed      [BH][M][D*D]       (compute type)
    float* zt;     // mixed normalisers [BH][M][D]  (fp32)
    Geo g;
    Tuning tune;
    int path;                     // MHLA_PATH_*
    const hipEvent_t* events;     // 4 events or nullptr
    hipStream_t stream;
};

// Enqueue the whole forward pass for one dtype.  Returns the first HIP error.
hipError_t run_bf16(const Launch& L);
hipError_t run_f32(const Launch& L);

}  // namespace mhla
