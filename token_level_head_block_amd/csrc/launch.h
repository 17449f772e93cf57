// launch.h -- internal launchers of the libmhla kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace mhla {

struct Tuning {
    int summary_waves;   // fp32 path: waves splitting the tokens of one block (1, 2, 4)
    int summary_pf;      // bf16 path: k-steps of K/V loads in flight per wave (1, 2)
    int apply_waves;     // waves splitting the tokens of one block in query_apply (1, 2, 4)
    int apply_pf;        // bf16 path: 16-token groups of Q loads in flight per wave (1, 2, 4)
    int nt_loads;        // bf16 path: non-temporal hint on the loads of k, v (summary kernel)
    int nt_apply;        // bf16 path: non-temporal hint on the loads of q (apply kernel)
    int mix_resident;    // bf16 path, M <= 256: persistent mixing kernel with W in registers
    int num_cus;         // compute units of the current device (persistent grid size)
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
    void* wb;      // bf16 path: W as bf16 [roundup(M,64)][roundup(M,32)], zero padded
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
