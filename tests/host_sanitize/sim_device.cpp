// sim_device.cpp -- a simulated device for the host-only sanitizer builds of
// the C-ABI layer (test infrastructure; never part of the library).
//
// The HIP calls fa_api.cpp makes are answered for four simulated devices:
// 0, 1 and 3 are gfx950 with 256 compute units, 2 is a gfx942 (the library
// must refuse it).  Device memory is host memory from malloc, so the
// sanitizers see every access.  The fa:: launchers stand in for the kernels:
// each checks the launch record for internal consistency and then reads every
// input byte and writes every output byte the real kernels would touch --
// q, k, v (or the paged caches through the block table), o, lse, and the
// split partials in the workspace.  A workspace or a buffer that the host
// layer sizes or points wrongly then shows up as an AddressSanitizer report.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "fa_launch.h"

namespace {

thread_local int g_current = 0;
std::atomic<long> g_live_allocs{0};

void die(const char *what)
{
    fprintf(stderr, "sim_device: inconsistent launch: %s\n", what);
    abort();
}

// Touch n bytes for reading: the sum keeps the reads from being optimised away.
volatile unsigned g_sink;
void read_bytes(const void *p, size_t n)
{
    if (!n) return;
    if (!p) die("null input");
    const unsigned char *b = static_cast<const unsigned char *>(p);
    unsigned s = 0;
    for (size_t i = 0; i < n; i += 61) s += b[i];
    s += b[n - 1];
    g_sink = g_sink + s;
}

void write_bytes(void *p, size_t n)
{
    if (!n) return;
    if (!p) die("null output");
    memset(p, 0x5a, n);
}

size_t rows(const fa::Launch &L) { return (size_t)L.B * L.Hq * L.Sq; }

void write_o_lse(const fa::Launch &L)
{
    write_bytes(L.o, rows(L) * L.D * (L.o_f32 ? 4 : 2));
    if (L.lse) write_bytes(L.lse, rows(L) * sizeof(float));
}

void write_partials(const fa::Launch &L)
{
    if (L.num_splits <= 1) return;
    if (!L.part_o || !L.part_lse) die("split launch without a workspace");
    if (L.part_lse != L.part_o + (size_t)L.num_splits * rows(L) * L.D)
        die("part_lse does not follow part_o");
    write_bytes(L.part_o, (size_t)L.num_splits * rows(L) * L.D * sizeof(float));
    write_bytes(L.part_lse, (size_t)L.num_splits * rows(L) * sizeof(float));
}

alignas(256) unsigned char g_scratch[fa::kStaticScratchBytes];

}  // namespace

extern "C" {

hipError_t hipGetDevice(int *device)
{
    if (getenv("SIM_NO_DEVICE")) return hipErrorNoDevice;
    *device = g_current;
    return hipSuccess;
}

hipError_t hipSetDevice(int device)
{
    if (device < 0 || device > 3) return hipErrorInvalidDevice;
    g_current = device;
    return hipSuccess;
}

hipError_t hipGetDeviceProperties(hipDeviceProp_t *prop, int device)
{
    if (device < 0 || device > 3) return hipErrorInvalidDevice;
    memset(prop, 0, sizeof(*prop));
    snprintf(prop->name, sizeof(prop->name), "simulated device %d", device);
    snprintf(prop->gcnArchName, sizeof(prop->gcnArchName), "%s",
             device == 2 ? "gfx942:sramecc+:xnack-" : "gfx950:sramecc+:xnack-");
    prop->multiProcessorCount = 256;
    return hipSuccess;
}

const char *hipGetErrorString(hipError_t e)
{
    switch (e) {
    case hipSuccess: return "hipSuccess";
    case hipErrorInvalidValue: return "hipErrorInvalidValue";
    case hipErrorOutOfMemory: return "hipErrorOutOfMemory";
    case hipErrorNoDevice: return "hipErrorNoDevice";
    case hipErrorInvalidDevice: return "hipErrorInvalidDevice";
    default: return "hipError (simulated)";
    }
}

hipError_t hipMalloc(void **ptr, size_t size)
{
    if (getenv("SIM_FAIL_MALLOC")) return hipErrorOutOfMemory;
    void *p = nullptr;
    if (posix_memalign(&p, 256, size ? size : 1) != 0) return hipErrorOutOfMemory;
    *ptr = p;
    ++g_live_allocs;
    return hipSuccess;
}

hipError_t hipFree(void *ptr)
{
    if (ptr) {
        free(ptr);
        --g_live_allocs;
    }
    return hipSuccess;
}

long sim_live_allocations(void) { return g_live_allocs.load(); }

}  // extern "C"

namespace fa {

bool prefill_cfg_ok(int D, int bn, int nw, int nr)
{
    static const int cfgs[][4] = {{128, 64, 8, 1}, {128, 64, 4, 1}, {128, 32, 4, 1},
                                  {128, 32, 8, 1}, {128, 64, 4, 2}, {64, 64, 8, 1},
                                  {64, 64, 4, 1},  {64, 32, 4, 1},  {64, 64, 4, 2},
                                  {256, 32, 4, 1}, {64, 32, 2, 1},  {128, 32, 2, 1}};
    for (const auto &c : cfgs)
        if (c[0] == D && c[1] == bn && c[2] == nw && c[3] == nr) return true;
    return false;
}

bool prefill_pp_ok(int D, int stages) { return (D == 64 || D == 128) && (stages == 4 || stages == 5); }

hipError_t static_scratch_ptr(int dev, void **out)
{
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    *out = g_scratch;
    return hipSuccess;
}

hipError_t launch_prefill(const Launch &L)
{
    if (L.grid < 1) die("prefill grid < 1");
    if (L.prefill_pp ? !prefill_pp_ok(L.D, L.prefill_pp)
                     : !prefill_cfg_ok(L.D, L.prefill_bn, L.prefill_nw, L.prefill_nr))
        die("prefill configuration not compiled");
    read_bytes(L.q, rows(L) * L.D * 2);
    read_bytes(L.k, (size_t)L.B * L.Sk * L.Hkv * L.D * 2);
    read_bytes(L.v, (size_t)L.B * L.Sk * L.Hkv * L.D * 2);
    write_o_lse(L);
    return hipSuccess;
}

hipError_t launch_decode(const Launch &L)
{
    if (L.num_splits < 1 || L.split_len < 1 || L.split_len % kDecodeBN)
        die("decode split plan");
    if ((long)L.num_splits * L.split_len < L.Sk || (long)(L.num_splits - 1) * L.split_len >= L.Sk)
        die("splits do not cover the keys exactly once");
    if (L.grid != L.B * L.Hkv * L.num_splits) die("decode grid");
    read_bytes(L.q, rows(L) * L.D * 2);
    read_bytes(L.k, (size_t)L.B * L.Sk * L.Hkv * L.D * 2);
    read_bytes(L.v, (size_t)L.B * L.Sk * L.Hkv * L.D * 2);
    write_partials(L);
    write_o_lse(L);
    return hipSuccess;
}

hipError_t launch_decode_paged(const Launch &L, const PagedLaunch &P)
{
    if (P.balanced) {
        // length-balanced ranges: range_cap of them, each with its KV heads
        if (L.grid != L.Hkv * P.range_cap || P.len_min < kDecodeBN || P.len_max < P.len_min ||
            P.len_min % kDecodeBN || P.len_max % kDecodeBN || P.slots < 1)
            die("balanced paged plan");
        if (P.range_cap < 1 || (long)P.range_cap * L.Hkv >= (1L << 31))
            die("range capacity");
        const size_t prow = (size_t)P.range_cap * L.Hq * L.Sq;
        if (!L.part_o || L.part_lse != L.part_o + prow * L.D) die("balanced partials");
        read_bytes(P.table, (size_t)L.B * P.max_pages * sizeof(int));
        read_bytes(P.seq_lens, (size_t)L.B * sizeof(int));
        write_bytes(L.part_o, prow * L.D * sizeof(float));
        write_bytes(L.part_lse, prow * sizeof(float));
        write_bytes(L.part_lse + prow, (size_t)2 * L.B * sizeof(int));   // range table
        write_o_lse(L);
        return hipSuccess;
    }
    if (L.num_splits < 1 || L.grid != L.B * L.Hkv * L.num_splits) die("paged grid");
    read_bytes(P.table, (size_t)L.B * P.max_pages * sizeof(int));
    read_bytes(P.seq_lens, (size_t)L.B * sizeof(int));
    const size_t page_bytes = (size_t)P.page_size * L.Hkv * L.D * 2;
    read_bytes(L.k, (size_t)P.num_pages * page_bytes);
    read_bytes(L.v, (size_t)P.num_pages * page_bytes);
    read_bytes(L.q, rows(L) * L.D * 2);
    write_partials(L);
    write_o_lse(L);
    return hipSuccess;
}

hipError_t launch_prefill_fp8(const Launch &L, float v_descale)
{
    if (L.D != 128 || (L.prefill_nw != 4 && L.prefill_nw != 8) || !(v_descale > 0.0f))
        die("fp8 launch");
    read_bytes(L.q, rows(L) * L.D);
    read_bytes(L.k, (size_t)L.B * L.Sk * L.Hkv * L.D);
    read_bytes(L.v, (size_t)L.B * L.Sk * L.Hkv * L.D);
    write_o_lse(L);
    return hipSuccess;
}

hipError_t launch_bwd(const BwdLaunch &L)
{
    const size_t nq = (size_t)L.B * L.Sq * L.Hq * L.D, nk = (size_t)L.B * L.Sk * L.Hkv * L.D;
    const size_t nr = (size_t)L.B * L.Hq * L.Sq;
    if (L.grid_dkdv < 1 || L.grid_dq < 1) die("backward grids");
    read_bytes(L.q, nq * 2);
    read_bytes(L.o, nq * 2);
    read_bytes(L.dout, nq * 2);
    read_bytes(L.k, nk * 2);
    read_bytes(L.v, nk * 2);
    read_bytes(L.lse, nr * sizeof(float));
    write_bytes(L.delta, 2 * nr * sizeof(float));
    write_bytes(L.dq, nq * 2);
    write_bytes(L.dk, nk * 2);
    write_bytes(L.dv, nk * 2);
    return hipSuccess;
}

}  // namespace fa
