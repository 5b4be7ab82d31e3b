// fa_launch.h -- internal interface between the C-ABI layer (fa_api.cpp) and
// the kernel launchers (fa_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace fa {

// Prefill tile configurations: waves per workgroup (32 query rows each) and
// keys per K/V tile; three tiles of K and V live in LDS at once.
constexpr int kPrefillStages = 3;
inline int prefill_lds_bytes(int D, int bn) { return kPrefillStages * 2 * bn * D * 2; }
inline bool prefill_cfg_ok(int D, int bn, int nw)
{
    if (D == 128) return (bn == 64 && (nw == 4 || nw == 8)) || (bn == 32 && (nw == 4 || nw == 8));
    return (bn == 64 && (nw == 4 || nw == 8)) || (bn == 32 && nw == 4);
}
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
    int prefill_bn;      // prefill: keys per tile
    int prefill_nw;      // prefill: waves per workgroup
    hipStream_t stream;
};

hipError_t launch_prefill(const Launch &L);
hipError_t launch_decode(const Launch &L);  // split kernel, then the merge pass if splits > 1

}  // namespace fa
