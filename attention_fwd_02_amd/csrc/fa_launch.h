// fa_launch.h -- internal interface between the C-ABI layer (fa_api.cpp) and
// the kernel launchers (fa_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace fa {

// Query rows per prefill workgroup (4 waves x 32 rows) and keys per tile.
constexpr int kPrefillBM = 128;
inline int prefill_block_n(int D) { return D == 64 ? 128 : 64; }
// Keys per tile of the split-key decode kernel; query rows it serves per KV head.
constexpr int kDecodeBN = 32;
constexpr int kDecodeRows = 32;

struct Launch {
    const void *q, *k, *v;
    void *o;
    float *lse;          // may be null
    float *part_o;       // split workspace: [splits][B][Hq][Sq][D] fp32
    float *part_lse;     //                  [splits][B][Hq][Sq]    fp32
    int B, Hq, Hkv, Sq, Sk, D;
    int causal;
    int o_f32;
    float scale;
    int num_splits;      // decode path
    int split_len;       // keys per split (multiple of kDecodeBN)
    int grid;            // prefill: persistent workgroups
    hipStream_t stream;
};

hipError_t launch_prefill(const Launch &L);
hipError_t launch_decode(const Launch &L);  // split kernel, then the merge pass if splits > 1

}  // namespace fa
