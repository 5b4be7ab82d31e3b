// fa_launch.h -- internal interface between the C-ABI layer (fa_api.cpp) and
// the kernel launchers (fa_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace fa {

// Prefill tile configurations: keys per K/V tile (bn), waves per workgroup
// (nw), 32-row query column blocks per wave (nr; 1 = two waves per SIMD,
// 2 = one wave per SIMD).  Three tiles of K and V live in LDS at once.
constexpr int kPrefillStages = 3;
inline int prefill_lds_bytes(int D, int bn) { return kPrefillStages * 2 * bn * D * 2; }
inline int prefill_waves_per_simd(int nr) { return nr == 1 ? 2 : 1; }
bool prefill_cfg_ok(int D, int bn, int nw, int nr);   // is this configuration compiled?
// Ping-pong prefill: 8 waves x 32 rows, 64-key tiles, two waves per SIMD in
// alternating MFMA and softmax phases; `stages` K/V tiles in the LDS ring.
constexpr int kPrefillPPWaves = 8;
constexpr int kPrefillPPBN = 64;
inline int prefill_pp_lds_bytes(int D, int stages) { return stages * 2 * kPrefillPPBN * D * 2; }
bool prefill_pp_ok(int D, int stages);
// Keys per tile of the split-key decode kernel; query rows it serves per KV
// head; depth of its LDS ring (tiles: one being read, the rest in flight).
constexpr int kDecodeBN = 32;
constexpr int kDecodeRows = 32;
#ifndef FA_DECODE_STAGES
#define FA_DECODE_STAGES 3
#endif
constexpr int kDecodeStages = FA_DECODE_STAGES;
// At D = 256 the decode kernels keep K and V in rings of their own, three K
// tiles and two V tiles (80 KiB: two workgroups per CU).
constexpr int kDecodeKStages256 = 3;
constexpr int kDecodeVStages256 = 2;
inline int decode_lds_bytes(int D)
{
    return D >= 256 ? (kDecodeKStages256 + kDecodeVStages256) * kDecodeBN * D * 2
                    : kDecodeStages * 2 * kDecodeBN * D * 2;
}
// Paged decode: a wave keeps the page ids of its key range in this many
// VGPRs (64 pages each), which bounds the pages one split may touch.
constexpr int kPagedIdRegs = 4;
constexpr int kPagedMaxPagesPerSplit = 64 * kPagedIdRegs;
// The length-balanced paged cut keeps the sequences' lengths in four
// registers per wave: at most this many sequences (beyond: equal splits).
constexpr int kPagedBalancedMaxSeqs = 256;

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
    int prefill_nr;      // prefill: 32-row column blocks per wave
    int head_major;      // prefill: item order (1: head by head, 0: rank by rank)
    int prefill_pp;      // prefill: 0, or the ring depth (4 or 5) of the ping-pong kernel
    int prefill_pipe = 0;  // prefill: 1 = the pipelined 32-key kernel (head dim 128: 8 waves)
    int fp8_pipe = 0;    // FP8 prefill: 1 = the pipelined kernel (8 waves)
    hipStream_t stream;
};

// Static scratch of the allocation-free entry point: kStaticScratchBytes per
// device (the split partials of one call), address per device.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
constexpr int kMaxScratchDevices = 64;
hipError_t static_scratch_ptr(int dev, void **out);   // `dev` must be current

hipError_t launch_prefill(const Launch &L);
hipError_t launch_decode(const Launch &L);  // split kernel, then the merge pass if splits > 1

// Paged K/V cache: L.k / L.v are the caches [num_pages][page_size][Hkv][D];
// L.Sk is unused.
struct PagedLaunch {
    const int *table;     // [B][max_pages] device
    const int *seq_lens;  // [B] device
    int num_pages, page_size, max_pages;
    // length-balanced ranges: one common range length, chosen on the device
    // within [len_min, len_max] so that the (range, KV head) items about fill
    // `slots`; grid and workspace provide for range_cap ranges.  The
    // workspace holds the partials, then [B][2] ints (each sequence's first
    // range and range count, for the merge)
    int balanced;
    int slots, range_cap, len_min, len_max;
};
hipError_t launch_decode_paged(const Launch &L, const PagedLaunch &P);

// FP8 E4M3 prefill: L.q/k/v hold E4M3 codes, L.scale already includes the
// q and k descales; O is multiplied by v_descale.  64-key tiles, 32 rows per
// wave, L.prefill_nw waves (4 or 8) per workgroup, L.grid workgroups.  With
// L.fp8_pipe the pipelined kernel runs instead: 8 waves (two per SIMD) x 32
// rows, separate K and V rings (48 KiB).
constexpr int kFp8BN = 64;
inline int fp8_lds_bytes(int D) { return kPrefillStages * 2 * kFp8BN * D; }
hipError_t launch_prefill_fp8(const Launch &L, float v_descale);

// Backward: delta pass, then dK/dV (workgroups of kBwdKeysPerWG keys of one
// KV head) and dQ (kBwdRowsPerWG query rows of one head), all on L.stream.
constexpr int kBwdKeysPerWG = 128;   // 4 waves x 32 keys (8: 39 registers spilled at D = 128)
constexpr int kBwdRowsPerWG = 256;   // 8 waves x 32 rows
struct BwdLaunch {
    const void *q, *k, *v, *o, *dout;   // bf16
    const float *lse;                   // [B][Hq][Sq] from the forward
    float *delta;                       // workspace: delta, then LSE * log2 e, [B][Hq][Sq] each
    void *dq, *dk, *dv;                 // bf16, layouts of q, k, v
    int B, Hq, Hkv, Sq, Sk, D, causal;
    float scale;
    int grid_dkdv, grid_dq;
    hipStream_t stream;
};
hipError_t launch_bwd(const BwdLaunch &L);

}  // namespace fa
