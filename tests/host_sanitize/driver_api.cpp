// driver_api.cpp -- exercises every entry point of include/fa.h on the
// simulated device (sim_device.cpp), under the host sanitizers: the five
// workloads of the suite and the paged, FP8, backward and allocation-free
// calls, every class of bad argument, the workspace paths (library-owned and
// grown, caller-provided, too small, allocation failure), a non-gfx950
// device, and (with "threads") eight threads calling at once on two devices.
// Exits 0 when every status is the expected one; the sanitizers abort it on
// any memory error, undefined behaviour or data race.

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <thread>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "fa.h"

extern "C" long sim_live_allocations(void);

namespace {

int g_fail = 0;

void expect(fa_status got, fa_status want, const char *what)
{
    if (got != want) {
        fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, (int)got, (int)want,
                fa_last_error());
        ++g_fail;
    }
}

// a "device" buffer of n bytes (host memory on the simulated device)
struct Buf {
    void *p = nullptr;
    explicit Buf(size_t n)
    {
        if (hipMalloc(&p, n) != hipSuccess) {
            fprintf(stderr, "hipMalloc(%zu) failed\n", n);
            exit(2);
        }
        memset(p, 0, n);
    }
    ~Buf() { hipFree(p); }
    Buf(const Buf &) = delete;
    Buf &operator=(const Buf &) = delete;
};

struct Shape {
    const char *name;
    int B, Hq, Hkv, Sq, Sk, D, causal;
    fa_dtype odt;
};

const Shape kShapes[] = {
    {"single head S=128 D=64, fp32 O", 1, 1, 1, 128, 128, 64, 0, FA_DTYPE_F32},
    {"causal B=2 H=8 S=1024 D=64", 2, 8, 8, 1024, 1024, 64, 1, FA_DTYPE_BF16},
    {"causal B=4 H=16 S=4096 D=128", 4, 16, 16, 4096, 4096, 128, 1, FA_DTYPE_BF16},
    {"decode B=32 Hq=32 Hkv=8 Sk=8192 D=128", 32, 32, 8, 1, 8192, 128, 0, FA_DTYPE_BF16},
    {"GQA B=1 Hq=32 Hkv=8 S=16384 D=128", 1, 32, 8, 16384, 16384, 128, 0, FA_DTYPE_BF16},
    {"causal B=2 H=16 S=4096 D=256", 2, 16, 16, 4096, 4096, 256, 1, FA_DTYPE_BF16},
    {"decode D=256", 32, 32, 8, 1, 8192, 256, 0, FA_DTYPE_BF16},
    {"ragged S=77x5 Sq>Sk causal", 2, 4, 2, 77, 5, 128, 1, FA_DTYPE_F32},
};

void forward_shapes()
{
    for (const Shape &s : kShapes) {
        const size_t qn = (size_t)s.B * s.Sq * s.Hq * s.D, kn = (size_t)s.B * s.Sk * s.Hkv * s.D;
        Buf q(qn * 2), k(kn * 2), v(kn * 2), o(qn * (s.odt == FA_DTYPE_F32 ? 4 : 2));
        Buf lse((size_t)s.B * s.Hq * s.Sq * 4);
        const float scale = 0.125f;
        fa_plan_info pi;
        expect(fa_plan(s.B, s.Hq, s.Hkv, s.Sq, s.Sk, s.D, s.causal, 0, &pi), FA_OK, s.name);
        const size_t ws = fa_workspace_size(s.B, s.Hq, s.Hkv, s.Sq, s.Sk, s.D, 0);
        if (ws != pi.workspace_bytes) {
            fprintf(stderr, "FAIL %s: workspace size %zu vs plan %zu\n", s.name, ws,
                    pi.workspace_bytes);
            ++g_fail;
        }
        // library-owned workspace, with and without LSE
        expect(fa_fwd_ex(q.p, k.p, v.p, o.p, (float *)lse.p, s.B, s.Hq, s.Hkv, s.Sq, s.Sk, s.D,
                         s.causal, scale, nullptr, s.odt, 0, nullptr, 0),
               FA_OK, s.name);
        expect(fa_fwd_ex(q.p, k.p, v.p, o.p, nullptr, s.B, s.Hq, s.Hkv, s.Sq, s.Sk, s.D, s.causal,
                         -scale, nullptr, s.odt, 0, nullptr, 0),
               FA_OK, s.name);
        if (s.odt == FA_DTYPE_BF16)
            expect(fa_fwd(q.p, k.p, v.p, o.p, (float *)lse.p, s.B, s.Hq, s.Hkv, s.Sq, s.Sk, s.D,
                          s.causal, scale, nullptr),
                   FA_OK, s.name);
        if (ws > 0) {
            // caller workspace: exact size works, one byte less is refused
            Buf w(ws);
            expect(fa_fwd_ex(q.p, k.p, v.p, o.p, (float *)lse.p, s.B, s.Hq, s.Hkv, s.Sq, s.Sk,
                             s.D, s.causal, scale, nullptr, s.odt, 0, w.p, ws),
                   FA_OK, s.name);
            expect(fa_fwd_ex(q.p, k.p, v.p, o.p, (float *)lse.p, s.B, s.Hq, s.Hkv, s.Sq, s.Sk,
                             s.D, s.causal, scale, nullptr, s.odt, 0, w.p, ws - 1),
                   FA_ERR_INVALID_ARG, s.name);
            // the allocation-free entry point, within its static buffer
            expect(fa_fwd_noalloc(q.p, k.p, v.p, o.p, (float *)lse.p, s.B, s.Hq, s.Hkv, s.Sq,
                                  s.Sk, s.D, s.causal, scale, nullptr, s.odt, 0),
                   ws <= (size_t(16) << 20) ? FA_OK : FA_ERR_UNSUPPORTED, s.name);
        }
        if ((size_t)s.Sq * (s.Hq / s.Hkv) <= 32) {
            // forced split counts, including more splits than tiles
            for (int ns : {1, 2, 7, 1000}) {
                fa_plan_info pf;
                expect(fa_plan(s.B, s.Hq, s.Hkv, s.Sq, s.Sk, s.D, s.causal, ns, &pf), FA_OK,
                       s.name);
                expect(fa_fwd_ex(q.p, k.p, v.p, o.p, (float *)lse.p, s.B, s.Hq, s.Hkv, s.Sq,
                                 s.Sk, s.D, s.causal, scale, nullptr, s.odt, ns, nullptr, 0),
                       FA_OK, s.name);
            }
        }
    }
}

void bad_arguments()
{
    Buf q(1 << 20), k(1 << 20), v(1 << 20), o(1 << 20), lse(1 << 16);
    char *qc = static_cast<char *>(q.p);
    float *l = static_cast<float *>(lse.p);
    struct Case {
        const char *what;
        fa_status want;
        fa_status got;
    } cases[] = {
        {"null q", FA_ERR_INVALID_ARG,
         fa_fwd(nullptr, k.p, v.p, o.p, l, 1, 1, 1, 8, 8, 64, 0, 1.0f, nullptr)},
        {"B = 0", FA_ERR_INVALID_ARG, fa_fwd(q.p, k.p, v.p, o.p, l, 0, 1, 1, 8, 8, 64, 0, 1.0f, nullptr)},
        {"Hq % Hkv", FA_ERR_INVALID_ARG, fa_fwd(q.p, k.p, v.p, o.p, l, 1, 3, 2, 8, 8, 64, 0, 1.0f, nullptr)},
        {"D = 96", FA_ERR_UNSUPPORTED, fa_fwd(q.p, k.p, v.p, o.p, l, 1, 1, 1, 8, 8, 96, 0, 1.0f, nullptr)},
        {"NaN scale", FA_ERR_INVALID_ARG,
         fa_fwd(q.p, k.p, v.p, o.p, l, 1, 1, 1, 8, 8, 64, 0, __builtin_nanf(""), nullptr)},
        {"causal = 2", FA_ERR_INVALID_ARG, fa_fwd(q.p, k.p, v.p, o.p, l, 1, 1, 1, 8, 8, 64, 2, 1.0f, nullptr)},
        {"misaligned q", FA_ERR_UNSUPPORTED,
         fa_fwd(qc + 2, k.p, v.p, o.p, l, 1, 1, 1, 8, 8, 64, 0, 1.0f, nullptr)},
        {"o dtype 7", FA_ERR_INVALID_ARG,
         fa_fwd_ex(q.p, k.p, v.p, o.p, l, 1, 1, 1, 8, 8, 64, 0, 1.0f, nullptr, (fa_dtype)7, 0, nullptr, 0)},
        {"negative splits", FA_ERR_INVALID_ARG,
         fa_fwd_ex(q.p, k.p, v.p, o.p, l, 1, 1, 1, 1, 8, 64, 0, 1.0f, nullptr, FA_DTYPE_BF16, -1, nullptr, 0)},
        {"splits on a prefill", FA_ERR_UNSUPPORTED,
         fa_fwd_ex(q.p, k.p, v.p, o.p, l, 1, 1, 1, 64, 8, 64, 0, 1.0f, nullptr, FA_DTYPE_BF16, 2, nullptr, 0)},
        {"K/V beyond 2 GiB per batch", FA_ERR_UNSUPPORTED,
         fa_fwd(q.p, k.p, v.p, o.p, l, 1, 8, 8, 1, 1 << 20, 128, 0, 1.0f, nullptr)},
        {"fp8 D = 64", FA_ERR_UNSUPPORTED,
         fa_fwd_fp8(q.p, k.p, v.p, o.p, l, 1, 1, 1, 8, 8, 64, 0, 1.0f, 1.0f, 1.0f, 1.0f, nullptr, FA_DTYPE_BF16)},
        {"fp8 zero descale", FA_ERR_INVALID_ARG,
         fa_fwd_fp8(q.p, k.p, v.p, o.p, l, 1, 1, 1, 8, 8, 128, 0, 1.0f, 0.0f, 1.0f, 1.0f, nullptr, FA_DTYPE_BF16)},
        {"bwd D = 256", FA_ERR_UNSUPPORTED,
         fa_bwd(q.p, k.p, v.p, o.p, o.p, l, q.p, k.p, v.p, 1, 1, 1, 8, 8, 256, 0, 1.0f, nullptr, nullptr, 0)},
        {"bwd null dout", FA_ERR_INVALID_ARG,
         fa_bwd(q.p, k.p, v.p, o.p, nullptr, l, q.p, k.p, v.p, 1, 1, 1, 8, 8, 64, 0, 1.0f, nullptr, nullptr, 0)},
        {"paged page size 24", FA_ERR_INVALID_ARG,
         fa_fwd_paged(q.p, k.p, v.p, (const int *)l, (const int *)l, o.p, l, 1, 1, 1, 1, 128, 4, 24, 4, 0,
                      1.0f, nullptr, FA_DTYPE_BF16, 0, nullptr, 0)},
        {"paged 64 query rows per KV head", FA_ERR_UNSUPPORTED,
         fa_fwd_paged(q.p, k.p, v.p, (const int *)l, (const int *)l, o.p, l, 1, 64, 1, 1, 128, 4, 16, 4, 0,
                      1.0f, nullptr, FA_DTYPE_BF16, 0, nullptr, 0)},
        {"plan null out", FA_ERR_INVALID_ARG, fa_plan(1, 1, 1, 8, 8, 64, 0, 0, nullptr)},
    };
    for (const Case &c : cases) {
        expect(c.got, c.want, c.what);
        if (c.got != FA_OK && strlen(fa_last_error()) == 0) {
            fprintf(stderr, "FAIL %s: empty fa_last_error\n", c.what);
            ++g_fail;
        }
    }
    if (fa_workspace_size(0, 1, 1, 1, 8, 64, 0) != 0 || fa_bwd_workspace_size(1, 3, 2, 8, 8, 64) != 0) {
        fprintf(stderr, "FAIL size queries of bad shapes must return 0\n");
        ++g_fail;
    }
}

void paged_fp8_bwd()
{
    // paged decode: B = 3, 16-key pages, lengths 300, 0, 77; unused entries -1
    const int B = 3, Hq = 8, Hkv = 2, D = 128, ps = 16, maxp = 19, npages = 40;
    Buf q((size_t)B * Hq * D * 2), kc((size_t)npages * ps * Hkv * D * 2),
        vc((size_t)npages * ps * Hkv * D * 2), o((size_t)B * Hq * D * 2), lse(B * Hq * 4);
    Buf table((size_t)B * maxp * 4), lens(B * 4);
    int *t = static_cast<int *>(table.p);
    for (int i = 0; i < B * maxp; ++i) t[i] = -1;
    const int len[3] = {300, 0, 77};
    int next = 0;
    for (int b = 0; b < B; ++b)
        for (int p = 0; p < (len[b] + ps - 1) / ps; ++p) t[b * maxp + p] = next++;
    memcpy(lens.p, len, sizeof(len));
    fa_plan_info pi;
    expect(fa_plan_paged(B, Hq, Hkv, 1, D, npages, ps, maxp, 0, &pi), FA_OK, "paged plan");
    expect(fa_fwd_paged(q.p, kc.p, vc.p, t, (const int *)lens.p, o.p, (float *)lse.p, B, Hq, Hkv, 1,
                        D, npages, ps, maxp, 0, 0.1f, nullptr, FA_DTYPE_BF16, 0, nullptr, 0),
           FA_OK, "paged decode");
    if (pi.workspace_bytes) {
        Buf w(pi.workspace_bytes);
        expect(fa_fwd_paged(q.p, kc.p, vc.p, t, (const int *)lens.p, o.p, (float *)lse.p, B, Hq,
                            Hkv, 1, D, npages, ps, maxp, 0, 0.1f, nullptr, FA_DTYPE_BF16, 0, w.p,
                            pi.workspace_bytes),
               FA_OK, "paged decode, caller workspace");
    }

    // FP8 prefill (one byte per element)
    {
        const int Bf = 2, H = 4, S = 700;
        Buf q8((size_t)Bf * S * H * 128), k8((size_t)Bf * S * H * 128), v8((size_t)Bf * S * H * 128);
        Buf of((size_t)Bf * S * H * 128 * 4), lf((size_t)Bf * H * S * 4);
        expect(fa_fwd_fp8(q8.p, k8.p, v8.p, of.p, (float *)lf.p, Bf, H, H, S, S, 128, 1, 0.088f,
                          0.01f, 0.02f, 0.03f, nullptr, FA_DTYPE_F32),
               FA_OK, "fp8 prefill");
    }

    // backward, library and caller workspace
    {
        const int Bb = 1, Hb = 4, Hk = 2, S = 600, Db = 128;
        const size_t nq = (size_t)Bb * S * Hb * Db, nk = (size_t)Bb * S * Hk * Db;
        Buf qb(nq * 2), kb(nk * 2), vb(nk * 2), ob(nq * 2), dob(nq * 2), lb((size_t)Bb * Hb * S * 4);
        Buf dq(nq * 2), dk(nk * 2), dv(nk * 2);
        expect(fa_bwd(qb.p, kb.p, vb.p, ob.p, dob.p, (const float *)lb.p, dq.p, dk.p, dv.p, Bb, Hb,
                      Hk, S, S, Db, 1, 0.088f, nullptr, nullptr, 0),
               FA_OK, "backward");
        const size_t ws = fa_bwd_workspace_size(Bb, Hb, Hk, S, S, Db);
        Buf w(ws);
        expect(fa_bwd(qb.p, kb.p, vb.p, ob.p, dob.p, (const float *)lb.p, dq.p, dk.p, dv.p, Bb, Hb,
                      Hk, S, S, Db, 1, 0.088f, nullptr, w.p, ws),
               FA_OK, "backward, caller workspace");
        expect(fa_bwd(qb.p, kb.p, vb.p, ob.p, dob.p, (const float *)lb.p, dq.p, dk.p, dv.p, Bb, Hb,
                      Hk, S, S, Db, 1, 0.088f, nullptr, w.p, ws - 4),
               FA_ERR_INVALID_ARG, "backward, workspace too small");
    }
}

void devices_and_allocation()
{
    Buf q(1 << 16), k(1 << 20), v(1 << 20), o(1 << 16), lse(1 << 12);
    // a gfx942 device is refused; device 3 (gfx950) works; back to 0
    hipSetDevice(2);
    expect(fa_fwd(q.p, k.p, v.p, o.p, (float *)lse.p, 1, 8, 2, 1, 512, 128, 0, 1.0f, nullptr),
           FA_ERR_UNSUPPORTED, "gfx942 device");
    hipSetDevice(3);
    expect(fa_fwd(q.p, k.p, v.p, o.p, (float *)lse.p, 1, 8, 2, 1, 512, 128, 0, 1.0f, nullptr),
           FA_OK, "second gfx950 device");
    expect(fa_release_workspace(), FA_OK, "release on device 3");
    hipSetDevice(0);
    // workspace allocation failure is reported, not crashed on
    expect(fa_release_workspace(), FA_OK, "release on device 0");
    setenv("SIM_FAIL_MALLOC", "1", 1);
    expect(fa_fwd(q.p, k.p, v.p, o.p, (float *)lse.p, 1, 8, 2, 1, 512, 128, 0, 1.0f, nullptr),
           FA_ERR_NOMEM, "hipMalloc failure");
    unsetenv("SIM_FAIL_MALLOC");
    setenv("FA_TEST_FAIL_ALLOC", "1", 1);
    expect(fa_fwd(q.p, k.p, v.p, o.p, (float *)lse.p, 1, 8, 2, 1, 512, 128, 0, 1.0f, nullptr),
           FA_ERR_NOMEM, "forced allocation failure");
    unsetenv("FA_TEST_FAIL_ALLOC");
    // no device at all: size queries still answer, calls report the HIP error
    setenv("SIM_NO_DEVICE", "1", 1);
    if (fa_workspace_size(32, 32, 8, 1, 8192, 128, 0) == 0) {
        fprintf(stderr, "FAIL workspace size without a device\n");
        ++g_fail;
    }
    expect(fa_fwd(q.p, k.p, v.p, o.p, (float *)lse.p, 1, 8, 2, 1, 512, 128, 0, 1.0f, nullptr),
           FA_ERR_HIP, "no device");
    unsetenv("SIM_NO_DEVICE");
}

void threads()
{
    // eight threads, two devices, decode shapes of different split workspace
    // sizes (the library-owned buffer grows under its lock) and plans
    std::vector<std::thread> ts;
    for (int t = 0; t < 8; ++t) {
        ts.emplace_back([t] {
            hipSetDevice(t % 2 ? 3 : 0);
            const int Sk = 1024 * (1 + t), B = 2 + t;
            const size_t qn = (size_t)B * 8 * 128, kn = (size_t)B * Sk * 2 * 128;
            Buf q(qn * 2), k(kn * 2), v(kn * 2), o(qn * 2), lse((size_t)B * 8 * 4);
            for (int it = 0; it < 20; ++it) {
                expect(fa_fwd(q.p, k.p, v.p, o.p, (float *)lse.p, B, 8, 2, 1, Sk, 128, 0, 0.1f,
                              nullptr),
                       FA_OK, "threaded decode");
                fa_plan_info pi;
                expect(fa_plan(B, 8, 2, 1, Sk, 128, 0, 0, &pi), FA_OK, "threaded plan");
                if (it % 7 == 3) expect(fa_release_workspace(), FA_OK, "threaded release");
            }
        });
    }
    for (auto &th : ts) th.join();
}

}  // namespace

int main(int argc, char **argv)
{
    const std::string what = argc > 1 ? argv[1] : "all";
    if (fa_version() <= 0) ++g_fail;
    if (what == "all") {
        forward_shapes();
        bad_arguments();
        paged_fp8_bwd();
        devices_and_allocation();
    }
    if (what == "all" || what == "threads") threads();
    hipSetDevice(0);
    fa_release_workspace();
    hipSetDevice(3);
    fa_release_workspace();
    if (sim_live_allocations() != 0) {
        fprintf(stderr, "FAIL %ld simulated device allocations still live\n",
                sim_live_allocations());
        ++g_fail;
    }
    printf("%s: %d failures\n", what.c_str(), g_fail);
    return g_fail ? 1 : 0;
}
