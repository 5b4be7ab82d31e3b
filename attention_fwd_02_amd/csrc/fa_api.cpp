// fa_api.cpp -- the C ABI declared in include/fa.h: argument checks, planning,
// split workspace, launches.  All device work is in fa_kernels.hip.
//
// The interface itself is this library's own: the pages name no API (the
// FlashAttention page of the Inference Cookbook lists a Python API page only
// by title).  Planning follows the waves-and-tail and persistent-scheduling
// discussion of "理解 H100：从硬件数据路径到 Nsight Compute 瓶颈分析" (occupancy
// and wave sections): the prefill grid is sized to the number of workgroups
// the CUs hold at once, and the decode path splits the key axis until the
// (batch, KV head, split) items fill the machine.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

thread_local std::string g_last_error;

fa_status fail(fa_status st, const std::string &msg)
{
    g_last_error = msg;
    return st;
}

// ---- device facts, queried once per device ---------------------------------
struct DeviceInfo {
    bool probed = false;
    bool supported = false;
    int cus = 0;
    std::string arch;
    // library-owned split workspace
    void *ws = nullptr;
    size_t ws_bytes = 0;
};

// One record per device index, at a fixed address for the life of the
// process: pointers handed out by device_info() stay valid whatever other
// threads probe later.
constexpr int kMaxDevices = 64;
std::mutex g_mu;
DeviceInfo g_dev[kMaxDevices];

// Fills in d (under g_mu) from the device's properties: no launch, no allocation.
hipError_t probe_locked(int dev, DeviceInfo &d)
{
    if (d.probed) return hipSuccess;
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return e;
    d.arch = prop.gcnArchName;
    d.cus = prop.multiProcessorCount;
    d.supported = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.probed = true;
    return hipSuccess;
}

fa_status device_info(int *dev_out, DeviceInfo **info_out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(FA_ERR_UNSUPPORTED, "device index beyond the library's table of 64");
    std::lock_guard<std::mutex> lk(g_mu);
    DeviceInfo &d = g_dev[dev];
    e = probe_locked(dev, d);
    if (e != hipSuccess)
        return fail(FA_ERR_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
    if (!d.supported) return fail(FA_ERR_UNSUPPORTED, "device architecture " + d.arch + " is not gfx950");
    *dev_out = dev;
    *info_out = &d;
    return FA_OK;
}

// The current device's compute-unit count for the pure size queries
// (fa_workspace_size, fa_plan, fa_plan_paged): the device property, read
// without launching anything, so that a size asked for before the first
// call equals what that call plans.  0 when no device is usable (the
// planner then assumes the MI355X's 256).
int query_cus()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::lock_guard<std::mutex> lk(g_mu);
    DeviceInfo &d = g_dev[dev];
    if (probe_locked(dev, d) != hipSuccess) return 0;
    return d.cus;
}

bool log_enabled()
{
    const char *s = getenv("FA_LOG");
    return s && s[0] == '1';
}

int env_int(const char *name, int dflt)
{
    const char *s = getenv(name);
    return (s && *s) ? atoi(s) : dflt;
}

// ---- argument checks (no HIP calls) ------------------------------------------
fa_status check_sizes(int B, int Hq, int Hkv, int Sq, int Sk, int D)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || D < 1)
        return fail(FA_ERR_INVALID_ARG, "every dimension must be >= 1");
    if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
    if (D != 64 && D != 128 && D != 256)
        return fail(FA_ERR_UNSUPPORTED, "head dim must be 64, 128 or 256");
    const int64_t q_elems = (int64_t)B * Sq * Hq * D;
    const int64_t k_elems = (int64_t)B * Sk * Hkv * D;
    if (q_elems >= (int64_t(1) << 40) || k_elems >= (int64_t(1) << 40))
        return fail(FA_ERR_UNSUPPORTED, "tensor too large");
    // K/V rows of one batch are addressed through 32-bit buffer byte offsets
    if ((int64_t)Sk * Hkv * D * 2 >= (int64_t(1) << 31))
        return fail(FA_ERR_UNSUPPORTED, "one batch of K or V exceeds 2 GiB");
    if ((int64_t)Sk + Sq >= (int64_t(1) << 30) || (int64_t)B * Hq >= (int64_t(1) << 30))
        return fail(FA_ERR_UNSUPPORTED, "sizes beyond 32-bit indexing");
    return FA_OK;
}

// ---- planning ------------------------------------------------------------------
struct Plan {
    int path = 0;        // 0 prefill, 1 split decode
    int num_splits = 1;
    int split_len = 0;
    int block_m = 0, block_n = 0;
    int grid = 0, items = 0;
    int prefill_bn = 0, prefill_nw = 0, prefill_nr = 1;
    int prefill_pp = 0;  // ring depth of the ping-pong kernel, 0 = not used
    int prefill_pipe = 0;  // the pipelined 32-key kernel at head dim 128 (8 waves)
    int head_major = 0;
    size_t ws_bytes = 0;
    size_t part_rows = 0;   // split partial rows in the workspace
    // paged decode with length-balanced ranges (see make_paged_plan)
    int balanced = 0;
    int slots = 0, range_cap = 0, len_min = 0, len_max = 0;
};

size_t split_ws_bytes(int B, int Hq, int Sq, int D, int ns)
{
    if (ns <= 1) return 0;
    return (size_t)ns * B * Hq * Sq * (size_t)(D + 1) * sizeof(float);
}

// cus = 0 when unknown (pure host query): use the MI355X count
fa_status make_plan(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int num_splits,
                    int cus, Plan *out)
{
    if (num_splits < 0) return fail(FA_ERR_INVALID_ARG, "num_splits must be >= 0");
    if (cus <= 0) cus = 256;
    Plan pl;
    const int group = Hq / Hkv;
    const int64_t rows_per_kv = (int64_t)Sq * group;
    const bool decode_ok = rows_per_kv <= fa::kDecodeRows;
    const int max_splits = (Sk + fa::kDecodeBN - 1) / fa::kDecodeBN;
    if (num_splits >= 1 && !decode_ok)
        return fail(FA_ERR_UNSUPPORTED,
                    "the split-key path serves at most 32 query rows per KV head (Sq * Hq / Hkv)");
    if (num_splits >= 1 || decode_ok) {
        pl.path = 1;
        int ns = num_splits;
        if (ns == 0) {
            ns = env_int("FA_NUM_SPLITS", 0);
            if (ns <= 0) {
                // enough (b, g, split) waves to fill every CU's resident slots
                // once (LDS ring and two waves per SIMD bound them), each
                // split >= 4 tiles; FA_DECODE_WAVES_PER_CU overrides the slots
                const int64_t bg = (int64_t)B * Hkv;
                int per_cu = std::min(8, (160 * 1024) / fa::decode_lds_bytes(D));
                per_cu = std::max(1, env_int("FA_DECODE_WAVES_PER_CU", per_cu));
                const int64_t want = ((int64_t)cus * per_cu + bg - 1) / bg;
                const int64_t by_len = std::max<int64_t>(1, Sk / (4 * fa::kDecodeBN));
                ns = (int)std::max<int64_t>(1, std::min<int64_t>(want, by_len));
            }
        }
        if (ns > max_splits) ns = max_splits;
        int len = (Sk + ns - 1) / ns;
        len = (len + fa::kDecodeBN - 1) / fa::kDecodeBN * fa::kDecodeBN;
        ns = (Sk + len - 1) / len;
        pl.num_splits = ns;
        pl.split_len = len;
        pl.block_m = fa::kDecodeRows;
        pl.block_n = fa::kDecodeBN;
        pl.items = B * Hkv * ns;
        pl.grid = pl.items;
        pl.ws_bytes = split_ws_bytes(B, Hq, Sq, D, ns);
        pl.part_rows = ns > 1 ? (size_t)ns * B * Hq * Sq : 0;
    } else {
        pl.path = 0;
        // tile configuration: 8 waves x 32 rows x 64 keys (two waves per
        // SIMD, K/V tiles shared by 256 query rows), or 4 waves x 64 rows
        // (one wave per SIMD); 4-wave, 32-key workgroups when 256-row items
        // leave CUs idle.  FA_PREFILL_BN / FA_PREFILL_NW / FA_PREFILL_NR
        // override (for measurements).
        int bn = 64, nw = 8, nr = 1;
        int pipe = 0;
        const int64_t m8 = (Sq + 255) / 256;
        // FA_PREFILL_PIPE: 0 = never the pipelined kernel at D = 128, 1 (the
        // default) = when 256-row items cover the CUs, 2 = always (tests)
        const int epipe = env_int("FA_PREFILL_PIPE", 1);
        if (D == 256) {
            // 32-key tiles (16 KiB per tile at D = 256: the three-stage ring
            // takes 96 KiB), 4 waves x 32 rows, one wave per SIMD (Q and O
            // alone take 192 registers per lane: two waves per SIMD spill)
            bn = 32;
            nw = 4;
        } else if (D == 128 && epipe == 2) {
            pipe = 1;
            bn = 32;
        } else if ((int64_t)B * Hq * m8 < cus) {
            nw = 4;
            bn = 32;
            // still fewer 128-row items than CUs: 64-row items (two waves),
            // so that every CU's LDS and L1 serve the same waves
            if ((int64_t)B * Hq * ((Sq + 127) / 128) < cus) nw = 2;
        } else if (D == 128 && epipe != 0) {
            // head dim 128: the pipelined 32-key kernel, 8 waves x 32 rows
            // (two waves per SIMD).  Measured against the 64-row kernel
            // (median of 30 interleaved calls): causal S = 1024 -10 %, 2048
            // -9 %, 4096 -4 %, 8192 -2 %, non-causal S = 4096 -4 %, GQA
            // S = 16384 equal.  FA_PREFILL_PIPE=0 restores the choice below.
            pipe = 1;
            bn = 32;
        } else if (!causal || Sq >= 2048) {
            // 64 rows per wave: faster wherever most tiles take its pipelined
            // body (non-causal, or causal rows of 2048 and more); shorter
            // causal rows spend too much of their time on diagonal tiles
            nw = 4;
            nr = 2;
        }
        const int ebn = env_int("FA_PREFILL_BN", 0), enw = env_int("FA_PREFILL_NW", 0);
        const int enr = env_int("FA_PREFILL_NR", 1);
        if (ebn > 0 && enw > 0 && fa::prefill_cfg_ok(D, ebn, enw, enr)) {
            bn = ebn;
            nw = enw;
            nr = enr;
            pipe = 0;
        }
        // the ping-pong kernel (8 waves x 32 rows, two per SIMD in opposite
        // MFMA / softmax phases, D = 64 or 128) only on request:
        // FA_PREFILL_PP = 4 / 5 (its ring depth)
        int pp = 0;
        const int epp = env_int("FA_PREFILL_PP", -1);
        if (epp == 0 || (epp > 0 && fa::prefill_pp_ok(D, epp))) pp = epp;
        if (ebn > 0 && enw > 0 && fa::prefill_cfg_ok(D, ebn, enw, enr)) pp = 0;
        if (pp) {
            bn = fa::kPrefillPPBN;
            nw = fa::kPrefillPPWaves;
            nr = 1;
            pipe = 0;
        }
        pl.prefill_pipe = pipe;
        const int bm = 32 * nw * nr;
        pl.block_m = bm;
        pl.block_n = bn;
        pl.prefill_bn = bn;
        pl.prefill_nw = nw;
        pl.prefill_nr = nr;
        pl.prefill_pp = pp;
        const int64_t items = (int64_t)B * Hq * ((Sq + bm - 1) / bm);
        if (items >= (int64_t(1) << 31)) return fail(FA_ERR_UNSUPPORTED, "too many work items");
        // workgroups a CU holds at once: LDS (160 KiB) and the waves per SIMD
        // the configuration's register budget allows (4 SIMDs per CU)
        int wg_per_cu = pp ? std::min((160 * 1024) / fa::prefill_pp_lds_bytes(D, pp), 1)
                           : std::min((160 * 1024) / fa::prefill_lds_bytes(D, bn),
                                      4 * fa::prefill_waves_per_simd(nr) / nw);
        wg_per_cu = std::max(1, std::min(wg_per_cu, env_int("FA_WG_PER_CU", wg_per_cu)));
        int64_t grid = std::min<int64_t>(items, (int64_t)cus * wg_per_cu);
        if (env_int("FA_PERSISTENT", 1) == 0) grid = items;
        // causal: head-major item order (measured faster, most for short
        // sequences: more of an XCD's workgroups share one head's K/V at a
        // time); non-causal: rank-major.  FA_HEAD_MAJOR overrides.
        pl.head_major = env_int("FA_HEAD_MAJOR", causal ? 1 : 0) != 0;
        pl.items = (int)items;
        pl.grid = (int)grid;
    }
    *out = pl;
    return FA_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Point L's split partials at the caller's workspace (checked against
// `need`) or at the device's library-owned buffer, grown on demand.  `lk`
// (on g_mu) stays locked while the launch uses the library buffer.
fa_status attach_workspace(DeviceInfo *info, void *workspace, size_t workspace_bytes, size_t need,
                           size_t part_rows, std::unique_lock<std::mutex> &lk, fa::Launch *L)
{
    void *ws = workspace;
    if (ws) {
        if (workspace_bytes < need)
            return fail(FA_ERR_INVALID_ARG, "workspace_bytes is smaller than the workspace size");
    } else {
        lk.lock();
        const char *force_fail = getenv("FA_TEST_FAIL_ALLOC");
        if (force_fail && force_fail[0] == '1')
            return fail(FA_ERR_NOMEM, "workspace allocation failed (forced by FA_TEST_FAIL_ALLOC)");
        if (info->ws_bytes < need) {
            if (info->ws) {
                // hipFree waits for the device, so work still queued on
                // any stream with the old buffer finishes first
                (void)hipFree(info->ws);
                info->ws = nullptr;
                info->ws_bytes = 0;
            }
            void *p = nullptr;
            hipError_t e = hipMalloc(&p, need);
            if (e != hipSuccess || !p)
                return fail(FA_ERR_NOMEM, std::string("workspace hipMalloc: ") + hipGetErrorString(e));
            info->ws = p;
            info->ws_bytes = need;
        }
        ws = info->ws;
    }
    L->part_o = static_cast<float *>(ws);
    L->part_lse = L->part_o + part_rows * L->D;
    return FA_OK;
}

// ---- paged K/V cache ---------------------------------------------------------
fa_status check_paged(int B, int Hq, int Hkv, int Sq, int D, int num_pages, int page_size,
                      int max_pages)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || D < 1 || num_pages < 1 || max_pages < 1)
        return fail(FA_ERR_INVALID_ARG, "every dimension must be >= 1");
    if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
    if (page_size < 16 || (page_size & (page_size - 1)) != 0)
        return fail(FA_ERR_INVALID_ARG, "page_size must be a power of two >= 16");
    if (D != 64 && D != 128 && D != 256)
        return fail(FA_ERR_UNSUPPORTED, "head dim must be 64, 128 or 256");
    if ((int64_t)Sq * (Hq / Hkv) > fa::kDecodeRows)
        return fail(FA_ERR_UNSUPPORTED,
                    "the paged path serves at most 32 query rows per KV head (Sq * Hq / Hkv)");
    // one page is addressed through 32-bit buffer byte offsets
    if ((int64_t)page_size * Hkv * D * 2 >= (int64_t(1) << 31))
        return fail(FA_ERR_UNSUPPORTED, "one cache page exceeds 2 GiB");
    if ((int64_t)max_pages * page_size + Sq >= (int64_t(1) << 30) ||
        (int64_t)B * max_pages >= (int64_t(1) << 31) || (int64_t)B * Hq * Sq >= (int64_t(1) << 30))
        return fail(FA_ERR_UNSUPPORTED, "sizes beyond 32-bit indexing");
    return FA_OK;
}

// Two ways to cut the keys of the paged decode.
//
// Length-balanced ranges (the automatic choice, num_splits = 0): every
// sequence's keys are cut into ranges of one common length L that the
// kernels derive on the device from the lengths: the shortest (at least 4
// tiles) for which the (range, KV head) items fit the CUs' resident slots in
// one round, at most len_max, the longest range whose pages fit the kernel's
// page-id registers.  A long sequence gets more ranges than a short one.  The
// host only bounds the count: range_cap = max(slots / Hkv, B * ceil(capacity /
// len_max)) ranges (grid and workspace) always suffice.  The merge always runs.
//
// Equal splits (num_splits >= 1, or FA_NUM_SPLITS, or FA_PAGED_BALANCED=0,
// or more than kPagedBalancedMaxSeqs sequences):
// each sequence's keys are cut into num_splits equal ranges (multiples of
// the tile).  The automatic count is sized for the table's capacity like the
// contiguous decode, then raised until one range touches at most
// kPagedMaxPagesPerSplit pages.
fa_status make_paged_plan(int B, int Hkv, int page_size, int max_pages, int D, int num_splits,
                          int cus, int Hq, int Sq, Plan *out)
{
    if (num_splits < 0) return fail(FA_ERR_INVALID_ARG, "num_splits must be >= 0");
    if (cus <= 0) cus = 256;
    const int64_t cap = (int64_t)max_pages * page_size;
    const int max_splits = (int)((cap + fa::kDecodeBN - 1) / fa::kDecodeBN);
    int per_cu = std::min(8, (160 * 1024) / fa::decode_lds_bytes(D));
    per_cu = std::max(1, env_int("FA_DECODE_WAVES_PER_CU", per_cu));
    int ns = num_splits;
    // (range counts are 32-bit on the device: ranges are at least 4 tiles)
    const bool count_fits =
        (int64_t)B * ((cap + 4 * fa::kDecodeBN - 1) / (4 * fa::kDecodeBN)) < (int64_t(1) << 31);
    if (ns == 0 && env_int("FA_NUM_SPLITS", 0) <= 0 && env_int("FA_PAGED_BALANCED", 1) != 0 &&
        B <= fa::kPagedBalancedMaxSeqs && count_fits) {
        const int64_t slots = (int64_t)cus * per_cu;
        const int64_t len_min = 4 * fa::kDecodeBN;
        const int64_t len_max =
            std::max<int64_t>(len_min, (int64_t)(fa::kPagedMaxPagesPerSplit - 1) * page_size /
                                           fa::kDecodeBN * fa::kDecodeBN);
        const int64_t range_cap = std::max<int64_t>(std::max<int64_t>(1, slots / Hkv),
                                                    (int64_t)B * ((cap + len_max - 1) / len_max));
        if (range_cap * Hkv >= (int64_t(1) << 31) || slots >= (int64_t(1) << 31))
            return fail(FA_ERR_UNSUPPORTED, "too many work items");
        Plan pl;
        pl.path = 1;
        pl.num_splits = 0;   // per sequence, on the device
        pl.split_len = 0;
        pl.block_m = fa::kDecodeRows;
        pl.block_n = fa::kDecodeBN;
        pl.items = (int)(range_cap * Hkv);
        pl.grid = pl.items;
        pl.part_rows = (size_t)range_cap * Hq * Sq;
        // partials, then each sequence's (first range, range count)
        pl.ws_bytes = pl.part_rows * (size_t)(D + 1) * sizeof(float) + (size_t)2 * B * sizeof(int);
        pl.balanced = 1;
        pl.slots = (int)slots;
        pl.range_cap = (int)range_cap;
        pl.len_min = (int)len_min;
        pl.len_max = (int)len_max;
        *out = pl;
        return FA_OK;
    }
    if (ns == 0) {
        ns = env_int("FA_NUM_SPLITS", 0);
        if (ns <= 0) {
            const int64_t bg = (int64_t)B * Hkv;
            const int64_t want = ((int64_t)cus * per_cu + bg - 1) / bg;
            const int64_t by_len = std::max<int64_t>(1, cap / (4 * fa::kDecodeBN));
            ns = (int)std::max<int64_t>(1, std::min<int64_t>(want, by_len));
        }
    }
    if (ns > max_splits) ns = max_splits;
    auto pages_per_split = [&](int n) {
        int64_t len = (cap + n - 1) / n;
        len = (len + fa::kDecodeBN - 1) / fa::kDecodeBN * fa::kDecodeBN;
        return (len + page_size - 1) / page_size + 1;
    };
    while (ns < max_splits && pages_per_split(ns) > fa::kPagedMaxPagesPerSplit) ++ns;
    if (pages_per_split(ns) > fa::kPagedMaxPagesPerSplit)
        return fail(FA_ERR_UNSUPPORTED, "page_size too small for one split's page-id registers");
    Plan pl;
    pl.path = 1;
    pl.num_splits = ns;
    pl.split_len = 0;   // per sequence, on the device
    pl.block_m = fa::kDecodeRows;
    pl.block_n = fa::kDecodeBN;
    const int64_t items = (int64_t)B * Hkv * ns;
    if (items >= (int64_t(1) << 31)) return fail(FA_ERR_UNSUPPORTED, "too many work items");
    pl.items = (int)items;
    pl.grid = pl.items;
    pl.ws_bytes = split_ws_bytes(B, Hq, Sq, D, ns);
    pl.part_rows = ns > 1 ? (size_t)ns * B * Hq * Sq : 0;
    *out = pl;
    return FA_OK;
}

// The forward of fa_fwd_ex and fa_fwd_noalloc.  `static_ws`: the split
// partials go to this device's static scratch array instead of a caller or
// library-owned workspace, and nothing is allocated.
fa_status fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq,
                   int Hkv, int Sq, int Sk, int D, int causal, float scale, hipStream_t stream,
                   fa_dtype o_dtype, int num_splits, void *workspace, size_t workspace_bytes,
                   bool static_ws)
{
    g_last_error.clear();
    if (!q || !k || !v || !o) return fail(FA_ERR_INVALID_ARG, "q, k, v and o must not be NULL");
    fa_status st = check_sizes(B, Hq, Hkv, Sq, Sk, D);
    if (st != FA_OK) return st;
    if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (o_dtype != FA_DTYPE_BF16 && o_dtype != FA_DTYPE_F32)
        return fail(FA_ERR_INVALID_ARG, "o_dtype must be FA_DTYPE_BF16 or FA_DTYPE_F32");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        (lse && !aligned16(lse)))
        return fail(FA_ERR_UNSUPPORTED, "q, k, v, o and lse must be 16-byte aligned");
    if (workspace && !aligned16(workspace))
        return fail(FA_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
    if (num_splits < 0) return fail(FA_ERR_INVALID_ARG, "num_splits must be >= 0");
    {
        // size-only plan check before touching the device
        Plan pre;
        st = make_plan(B, Hq, Hkv, Sq, Sk, D, causal, num_splits, 0, &pre);
        if (st != FA_OK) return st;
    }

    int dev = 0;
    DeviceInfo *info = nullptr;
    st = device_info(&dev, &info);
    if (st != FA_OK) return st;

    Plan pl;
    st = make_plan(B, Hq, Hkv, Sq, Sk, D, causal, num_splits, info->cus, &pl);
    if (st != FA_OK) return st;
    if (static_ws && pl.ws_bytes > fa::kStaticScratchBytes)
        return fail(FA_ERR_UNSUPPORTED,
                    "the split plan needs " + std::to_string(pl.ws_bytes) +
                        " bytes of scratch; the static buffer of fa_fwd_noalloc holds " +
                        std::to_string(fa::kStaticScratchBytes) +
                        " (call fa_fwd_ex with a workspace instead)");

    fa::Launch L;
    L.q = q; L.k = k; L.v = v; L.o = o; L.lse = lse;
    L.part_o = nullptr; L.part_lse = nullptr;
    L.B = B; L.Hq = Hq; L.Hkv = Hkv; L.Sq = Sq; L.Sk = Sk; L.D = D;
    L.causal = causal;
    L.o_f32 = (o_dtype == FA_DTYPE_F32);
    L.scale = scale;
    L.num_splits = pl.num_splits;
    L.split_len = pl.split_len;
    L.grid = pl.grid;
    L.prefill_bn = pl.prefill_bn;
    L.prefill_nw = pl.prefill_nw;
    L.prefill_nr = pl.prefill_nr;
    L.prefill_pp = pl.prefill_pp;
    L.prefill_pipe = pl.prefill_pipe;
    L.head_major = pl.head_major;
    L.stream = stream;

    if (log_enabled())
        fprintf(stderr,
                "[fa] path=%s B=%d Hq=%d Hkv=%d Sq=%d Sk=%d D=%d causal=%d splits=%d "
                "split_len=%d block=%dx%d waves=%d grid=%d items=%d ws=%zu\n",
                pl.path ? "split-decode" : "prefill", B, Hq, Hkv, Sq, Sk, D, causal,
                pl.num_splits, pl.split_len, pl.block_m, pl.block_n,
                pl.path ? 1 : pl.prefill_nw, pl.grid, pl.items, pl.ws_bytes);

    hipError_t e;
    if (pl.path == 0) {
        e = fa::launch_prefill(L);
    } else if (static_ws) {
        if (pl.ws_bytes > 0) {
            void *ws = nullptr;
            e = fa::static_scratch_ptr(dev, &ws);
            if (e != hipSuccess)
                return fail(FA_ERR_HIP, std::string("hipGetSymbolAddress: ") + hipGetErrorString(e));
            L.part_o = static_cast<float *>(ws);
            L.part_lse = L.part_o + pl.part_rows * D;
        }
        e = fa::launch_decode(L);
    } else {
        std::unique_lock<std::mutex> lk(g_mu, std::defer_lock);
        if (pl.ws_bytes > 0) {
            st = attach_workspace(info, workspace, workspace_bytes, pl.ws_bytes, pl.part_rows,
                                  lk, &L);
            if (st != FA_OK) return st;
        }
        e = fa::launch_decode(L);
    }
    if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                    int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale,
                    hipStream_t stream, fa_dtype o_dtype, int num_splits, void *workspace,
                    size_t workspace_bytes)
{
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, causal, scale, stream, o_dtype,
                    num_splits, workspace, workspace_bytes, false);
}

fa_status fa_fwd_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                         int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale,
                         hipStream_t stream, fa_dtype o_dtype, int num_splits)
{
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, causal, scale, stream, o_dtype,
                    num_splits, nullptr, 0, true);
}

fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq,
                 int Hkv, int Sq, int Sk, int D, int causal, float scale, hipStream_t stream)
{
    return fa_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, causal, scale, stream,
                     FA_DTYPE_BF16, 0, nullptr, 0);
}

size_t fa_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int D, int num_splits)
{
    if (check_sizes(B, Hq, Hkv, Sq, Sk, D) != FA_OK) return 0;
    const int cus = query_cus();
    Plan pl;
    // the workspace depends on the split plan only, which ignores causality
    if (make_plan(B, Hq, Hkv, Sq, Sk, D, 0, num_splits, cus, &pl) != FA_OK) return 0;
    return pl.ws_bytes;
}

fa_status fa_plan(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int num_splits,
                  fa_plan_info *out)
{
    g_last_error.clear();
    if (!out) return fail(FA_ERR_INVALID_ARG, "out must not be NULL");
    fa_status st = check_sizes(B, Hq, Hkv, Sq, Sk, D);
    if (st != FA_OK) return st;
    const int cus = query_cus();
    Plan pl;
    st = make_plan(B, Hq, Hkv, Sq, Sk, D, causal, num_splits, cus, &pl);
    if (st != FA_OK) return st;
    out->path = pl.path;
    out->num_splits = pl.num_splits;
    out->block_m = pl.block_m;
    out->block_n = pl.block_n;
    out->grid = pl.grid;
    out->work_items = pl.items;
    out->workspace_bytes = pl.ws_bytes;
    out->waves = pl.path == 0 ? pl.prefill_nw : 1;
    out->rows_per_wave = pl.path == 0 ? 32 * pl.prefill_nr : 0;
    return FA_OK;
}

fa_status fa_fwd_paged(const void *q, const void *k_cache, const void *v_cache,
                       const int *block_table, const int *seq_lens, void *o, float *lse, int B,
                       int Hq, int Hkv, int Sq, int D, int num_pages, int page_size,
                       int max_pages, int causal, float scale, hipStream_t stream,
                       fa_dtype o_dtype, int num_splits, void *workspace, size_t workspace_bytes)
{
    g_last_error.clear();
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o)
        return fail(FA_ERR_INVALID_ARG,
                    "q, k_cache, v_cache, block_table, seq_lens and o must not be NULL");
    fa_status st = check_paged(B, Hq, Hkv, Sq, D, num_pages, page_size, max_pages);
    if (st != FA_OK) return st;
    if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (o_dtype != FA_DTYPE_BF16 && o_dtype != FA_DTYPE_F32)
        return fail(FA_ERR_INVALID_ARG, "o_dtype must be FA_DTYPE_BF16 or FA_DTYPE_F32");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
        (lse && !aligned16(lse)) || (workspace && !aligned16(workspace)))
        return fail(FA_ERR_UNSUPPORTED,
                    "q, k_cache, v_cache, o, lse and workspace must be 16-byte aligned");
    if (((uintptr_t)block_table & 3u) || ((uintptr_t)seq_lens & 3u))
        return fail(FA_ERR_UNSUPPORTED, "block_table and seq_lens must be 4-byte aligned");
    if (num_splits < 0) return fail(FA_ERR_INVALID_ARG, "num_splits must be >= 0");
    {
        Plan pre;
        st = make_paged_plan(B, Hkv, page_size, max_pages, D, num_splits, 0, Hq, Sq, &pre);
        if (st != FA_OK) return st;
    }

    int dev = 0;
    DeviceInfo *info = nullptr;
    st = device_info(&dev, &info);
    if (st != FA_OK) return st;
    Plan pl;
    st = make_paged_plan(B, Hkv, page_size, max_pages, D, num_splits, info->cus, Hq, Sq, &pl);
    if (st != FA_OK) return st;

    fa::Launch L;
    L.q = q; L.k = k_cache; L.v = v_cache; L.o = o; L.lse = lse;
    L.part_o = nullptr; L.part_lse = nullptr;
    L.B = B; L.Hq = Hq; L.Hkv = Hkv; L.Sq = Sq; L.Sk = 0; L.D = D;
    L.causal = causal;
    L.o_f32 = (o_dtype == FA_DTYPE_F32);
    L.scale = scale;
    L.num_splits = pl.num_splits;
    L.split_len = 0;
    L.grid = pl.grid;
    L.prefill_bn = L.prefill_nw = L.prefill_nr = 0;
    L.prefill_pp = 0;
    L.head_major = 0;
    L.stream = stream;
    fa::PagedLaunch P;
    P.table = block_table;
    P.seq_lens = seq_lens;
    P.num_pages = num_pages;
    P.page_size = page_size;
    P.max_pages = max_pages;
    P.balanced = pl.balanced;
    P.slots = pl.slots;
    P.range_cap = pl.range_cap;
    P.len_min = pl.len_min;
    P.len_max = pl.len_max;

    if (log_enabled())
        fprintf(stderr,
                "[fa] path=paged-decode B=%d Hq=%d Hkv=%d Sq=%d D=%d pages=%d page_size=%d "
                "max_pages=%d causal=%d splits=%d grid=%d ws=%zu\n",
                B, Hq, Hkv, Sq, D, num_pages, page_size, max_pages, causal, pl.num_splits,
                pl.grid, pl.ws_bytes);

    std::unique_lock<std::mutex> lk(g_mu, std::defer_lock);
    if (pl.ws_bytes > 0) {
        st = attach_workspace(info, workspace, workspace_bytes, pl.ws_bytes, pl.part_rows, lk, &L);
        if (st != FA_OK) return st;
    }
    hipError_t e = fa::launch_decode_paged(L, P);
    if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return FA_OK;
}

fa_status fa_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                     int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale,
                     float q_descale, float k_descale, float v_descale, hipStream_t stream,
                     fa_dtype o_dtype)
{
    g_last_error.clear();
    if (!q || !k || !v || !o) return fail(FA_ERR_INVALID_ARG, "q, k, v and o must not be NULL");
    fa_status st = check_sizes(B, Hq, Hkv, Sq, Sk, D);
    if (st != FA_OK) return st;
    if (D != 128) return fail(FA_ERR_UNSUPPORTED, "the FP8 path serves head dim 128");
    if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
    if (!(q_descale > 0.0f) || !(k_descale > 0.0f) || !(v_descale > 0.0f) ||
        !isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale))
        return fail(FA_ERR_INVALID_ARG, "descales must be finite and > 0");
    const float s_eff = scale * q_descale * k_descale;
    if (!isfinite(s_eff)) return fail(FA_ERR_INVALID_ARG, "scale * q_descale * k_descale overflows");
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (o_dtype != FA_DTYPE_BF16 && o_dtype != FA_DTYPE_F32)
        return fail(FA_ERR_INVALID_ARG, "o_dtype must be FA_DTYPE_BF16 or FA_DTYPE_F32");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        (lse && !aligned16(lse)))
        return fail(FA_ERR_UNSUPPORTED, "q, k, v, o and lse must be 16-byte aligned");

    int dev = 0;
    DeviceInfo *info = nullptr;
    st = device_info(&dev, &info);
    if (st != FA_OK) return st;

    // 32 rows per wave, 64-key tiles, 8 waves (two per SIMD, 256 registers
    // each): the pipelined kernel.  FA_FP8_PIPE=0 selects the earlier
    // unpipelined one, and FA_FP8_NW=4 its one-wave-per-SIMD form (measured
    // 1.7x slower on the causal S=4096 shape: no second wave fills the first's
    // stalls).
    const int nw = env_int("FA_FP8_NW", 8) == 4 ? 4 : 8;
    const int pipe = (nw == 8 && env_int("FA_FP8_PIPE", 1) != 0) ? 1 : 0;
    const int bm = 32 * nw;
    const int64_t items = (int64_t)B * Hq * ((Sq + bm - 1) / bm);
    if (items >= (int64_t(1) << 31)) return fail(FA_ERR_UNSUPPORTED, "too many work items");
    const int wg_per_cu = 1;
    const int64_t grid = std::min<int64_t>(items, (int64_t)info->cus * wg_per_cu);

    fa::Launch L;
    L.q = q; L.k = k; L.v = v; L.o = o; L.lse = lse;
    L.part_o = nullptr; L.part_lse = nullptr;
    L.B = B; L.Hq = Hq; L.Hkv = Hkv; L.Sq = Sq; L.Sk = Sk; L.D = D;
    L.causal = causal;
    L.o_f32 = (o_dtype == FA_DTYPE_F32);
    L.scale = s_eff;
    L.num_splits = 1;
    L.split_len = 0;
    L.grid = (int)grid;
    L.prefill_bn = fa::kFp8BN;
    L.prefill_nw = nw;
    L.prefill_nr = 1;
    L.prefill_pp = 0;
    L.fp8_pipe = pipe;
    L.head_major = env_int("FA_HEAD_MAJOR", causal ? 1 : 0) != 0;
    L.stream = stream;
    if (log_enabled())
        fprintf(stderr, "[fa] path=fp8-prefill B=%d Hq=%d Hkv=%d Sq=%d Sk=%d D=%d causal=%d "
                "waves=%d pipe=%d grid=%lld items=%lld\n", B, Hq, Hkv, Sq, Sk, D, causal, nw,
                pipe, (long long)grid, (long long)items);
    hipError_t e = fa::launch_prefill_fp8(L, v_descale);
    if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return FA_OK;
}

size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int D)
{
    if (check_sizes(B, Hq, Hkv, Sq, Sk, D) != FA_OK) return 0;
    return (size_t)2 * B * Hq * Sq * sizeof(float);
}

fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                 const float *lse, void *dq, void *dk, void *dv, int B, int Hq, int Hkv, int Sq,
                 int Sk, int D, int causal, float scale, hipStream_t stream, void *workspace,
                 size_t workspace_bytes)
{
    g_last_error.clear();
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
        return fail(FA_ERR_INVALID_ARG, "no pointer of fa_bwd may be NULL");
    fa_status st = check_sizes(B, Hq, Hkv, Sq, Sk, D);
    if (st != FA_OK) return st;
    if (D != 64 && D != 128) return fail(FA_ERR_UNSUPPORTED, "the backward serves head dims 64 and 128");
    // Q and dO tiles are addressed like K/V in the forward: 32-bit byte offsets per batch
    if ((int64_t)Sq * Hq * D * 2 >= (int64_t(1) << 31))
        return fail(FA_ERR_UNSUPPORTED, "one batch of q exceeds 2 GiB");
    if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
        !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
        (workspace && !aligned16(workspace)))
        return fail(FA_ERR_UNSUPPORTED, "every pointer of fa_bwd must be 16-byte aligned");
    const size_t need = (size_t)2 * B * Hq * Sq * sizeof(float);   // delta, LSE * log2 e

    int dev = 0;
    DeviceInfo *info = nullptr;
    st = device_info(&dev, &info);
    if (st != FA_OK) return st;

    fa::BwdLaunch L;
    L.q = q; L.k = k; L.v = v; L.o = o; L.dout = dout; L.lse = lse;
    L.dq = dq; L.dk = dk; L.dv = dv;
    L.B = B; L.Hq = Hq; L.Hkv = Hkv; L.Sq = Sq; L.Sk = Sk; L.D = D; L.causal = causal;
    L.scale = scale;
    L.stream = stream;
    // one workgroup per CU for both kernels (LDS rings of about 96 KiB)
    const int64_t items_kv = (int64_t)B * Hkv * ((Sk + fa::kBwdKeysPerWG - 1) / fa::kBwdKeysPerWG);
    const int64_t items_q = (int64_t)B * Hq * ((Sq + fa::kBwdRowsPerWG - 1) / fa::kBwdRowsPerWG);
    if (items_kv >= (int64_t(1) << 31) || items_q >= (int64_t(1) << 31))
        return fail(FA_ERR_UNSUPPORTED, "too many work items");
    L.grid_dkdv = (int)std::min<int64_t>(items_kv, info->cus);
    L.grid_dq = (int)std::min<int64_t>(items_q, info->cus);

    std::unique_lock<std::mutex> lk(g_mu, std::defer_lock);
    void *ws = workspace;
    if (ws) {
        if (workspace_bytes < need)
            return fail(FA_ERR_INVALID_ARG, "workspace_bytes is smaller than fa_bwd_workspace_size()");
    } else {
        lk.lock();
        if (info->ws_bytes < need) {
            if (info->ws) {
                (void)hipFree(info->ws);
                info->ws = nullptr;
                info->ws_bytes = 0;
            }
            void *pw = nullptr;
            hipError_t e = hipMalloc(&pw, need);
            if (e != hipSuccess || !pw)
                return fail(FA_ERR_NOMEM, std::string("workspace hipMalloc: ") + hipGetErrorString(e));
            info->ws = pw;
            info->ws_bytes = need;
        }
        ws = info->ws;
    }
    L.delta = static_cast<float *>(ws);
    if (log_enabled())
        fprintf(stderr, "[fa] path=backward B=%d Hq=%d Hkv=%d Sq=%d Sk=%d D=%d causal=%d "
                "grid_dkdv=%d grid_dq=%d\n", B, Hq, Hkv, Sq, Sk, D, causal, L.grid_dkdv, L.grid_dq);
    hipError_t e = fa::launch_bwd(L);
    if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return FA_OK;
}

fa_status fa_plan_paged(int B, int Hq, int Hkv, int Sq, int D, int num_pages, int page_size,
                        int max_pages, int num_splits, fa_plan_info *out)
{
    g_last_error.clear();
    if (!out) return fail(FA_ERR_INVALID_ARG, "out must not be NULL");
    fa_status st = check_paged(B, Hq, Hkv, Sq, D, num_pages, page_size, max_pages);
    if (st != FA_OK) return st;
    Plan pl;
    st = make_paged_plan(B, Hkv, page_size, max_pages, D, num_splits, query_cus(), Hq, Sq, &pl);
    if (st != FA_OK) return st;
    out->path = 2;
    out->num_splits = pl.num_splits;
    out->block_m = pl.block_m;
    out->block_n = pl.block_n;
    out->grid = pl.grid;
    out->work_items = pl.items;
    out->workspace_bytes = pl.ws_bytes;
    out->waves = 1;
    out->rows_per_wave = 0;
    return FA_OK;
}

const char *fa_last_error(void) { return g_last_error.c_str(); }

fa_status fa_release_workspace(void)
{
    std::lock_guard<std::mutex> lk(g_mu);
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) cur = -1;
    for (int d = 0; d < kMaxDevices; ++d) {
        if (!g_dev[d].ws) continue;
        if (hipSetDevice(d) == hipSuccess) (void)hipFree(g_dev[d].ws);
        g_dev[d].ws = nullptr;
        g_dev[d].ws_bytes = 0;
    }
    if (cur >= 0) (void)hipSetDevice(cur);
    return FA_OK;
}

int fa_version(void) { return 100; }

}  // extern "C"
