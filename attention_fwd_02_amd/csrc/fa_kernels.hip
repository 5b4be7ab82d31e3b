// fa_kernels.hip -- fused attention forward kernels for gfx950 (CDNA4, wave64).
//
// What is computed: O = softmax(scale * Q K^T [causal]) V and LSE per query
// row, never writing S or P to HBM.  The structure follows the FlashAttention
// forward main loop laid out in "SM80 内核实现对比" (Inference Cookbook): Q kept
// in registers for the whole key loop (section 5.3, Q_in_regs), K/V tiles
// staged through on-chip memory with a software pipeline (section 4.1), the
// S = Q K^T product, the online softmax, then P V with P taken from registers
// (section 5.2), and 16-byte global copies (section 2.1).  The online-softmax
// pieces -- row max, exp, row sum, rescale, causal mask -- are those named in
// "从 Volta/Turing、Ampere、Ada 到 Hopper：硬件、PTX 与 Kernel 编程范式演进",
// section "Attention 的瓶颈会在 Tensor Core 与 CUDA Core 之间迁移".
//
// What is CDNA4-specific (and differs from the pages' SM80/SM90 designs):
//  * Both products run on v_mfma_f32_32x32x16_bf16 in the transposed form
//    S^T = K Q^T and O^T = V^T P^T.  In the 32x32 accumulator layout a lane owns
//    one output column (here: one query) and 16 rows (keys, or head dims), so
//    the row max and row sum need a single cross-lane step (v_permlane32_swap)
//    instead of a shuffle tree, and the per-query rescale factor is lane-local.
//  * P never leaves registers: the S^T accumulator registers are reused as the
//    B operand of the PV MFMA.  The keys a lane holds there are not
//    contiguous, so the V tile is written to LDS transposed (V^T[d][key]) and
//    with the key index permuted inside each 16-key group (bits 2 and 3
//    swapped); summing over keys in a permuted order is exact.
//  * LDS rows are XOR-swizzled in 16-byte chunks so that the 32 rows read by
//    one ds_read_b128 fall on distinct banks.
//  * Prefill runs a persistent grid (two 256-thread workgroups per CU) that
//    walks (batch, head, query block) items in a snake order, longest causal
//    blocks first, and keeps all blocks of a head on one XCD so that their K/V
//    re-reads hit that XCD's L2.
//  * Decode (few query rows per KV head) runs a split-key kernel, one wave per
//    (batch, KV head, key range), which writes partial (O_s, LSE_s); a merge
//    pass combines them with log-sum-exp weights.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_launch.h"

namespace fa {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef float f32x16_t __attribute__((__vector_size__(64)));
typedef uint32_t u32x4_t __attribute__((__vector_size__(16)));
typedef uint32_t u32x2_t __attribute__((__vector_size__(8)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegInf = -__builtin_inff();
// Word 3 of a gfx9-family buffer descriptor: 32-bit data format, so that
// untyped dword loads are valid; out-of-range offsets return zero.
constexpr int kBufferFlags = 0x00020000;

struct Params {
    const uint16_t *q, *k, *v;
    void *o;
    float *lse;
    float *part_o, *part_lse;
    int B, Hq, Hkv, Sq, Sk;
    int group;        // Hq / Hkv
    int causal;
    int off;          // Sk - Sq: key j allowed for query i iff j <= i + off
    float c;          // |scale| * log2(e)
    uint32_t qflip;   // 0x80008000 when scale < 0 (Q is negated exactly instead)
    int n_mblocks;    // prefill: query blocks per head
    int domains;      // prefill: XCD scheduling domains (8 or 1)
    int num_splits, split_len;
};

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Combine a value with the one held by lane ^ 32 through a symmetric op.
__device__ __forceinline__ float max_halves(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_halves(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Position of key `key` (0..) inside a transposed V tile: bits 2 and 3 of the
// key index swap inside each 16-key group, so that the 8 keys lane-half h of
// the PV MFMA needs (keys 4h..4h+3 and 8+4h..8+4h+3 of the group) are adjacent.
__device__ __forceinline__ int vt_pos(int key)
{
    return (key & ~15) | ((key & 4) << 1) | ((key & 8) >> 1) | (key & 3);
}

__device__ __forceinline__ u32x4_t ld16(const uint16_t *p)
{
    return *reinterpret_cast<const u32x4_t *>(p);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    __bf16 x = (__bf16)a, y = (__bf16)b;  // round to nearest even (v_cvt_pk_bf16_f32)
    return (uint32_t)__builtin_bit_cast(uint16_t, x) |
           ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// ---------------------------------------------------------------------------
// One wave's share of a K/V tile held in LDS: S^T, online softmax, O^T += V^T P^T.
//
// K tile in LDS: Ks[key][D] bf16, 16-byte chunk c of row key stored at chunk
//   c ^ (key % KCH).  V tile: Vt[d][BN] bf16 (keys in vt_pos order), chunk c of
//   row d stored at c ^ (d % VCH).
// Lane (col, half): query column `col`; after the S^T MFMA its register r of
//   key block kb holds key kb*32 + 8*(r/4) + 4*half + (r%4).
// ---------------------------------------------------------------------------
template <int D, int BN>
struct WaveTile {
    static constexpr int KCH = D / 8;
    static constexpr int VCH = BN / 8;
    static constexpr int QS = D / 16;
    static constexpr int KB = BN / 32;
    static constexpr int DB = D / 32;
    static constexpr int PS = BN / 16;

    // mask_mode: 0 = every key allowed; 1 = per element check
    template <bool MASK>
    __device__ __forceinline__ static void step(const uint16_t *__restrict__ Ks,
                                                const uint16_t *__restrict__ Vt,
                                                const bf16x8_t (&qf)[QS], f32x16_t (&o)[DB],
                                                float &m_run, float &l_run, float c, int col,
                                                int half, int key0, int key_end, int lim)
    {
        // ---- S^T = K Q^T over this tile's BN keys ----
        f32x16_t s[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16_t{};
#pragma unroll
        for (int st = 0; st < QS; ++st) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int key = kb * 32 + col;
                const int ch = 2 * st + half;
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(
                    Ks + key * D + ((ch ^ (key % KCH)) * 8));
                s[kb] = mfma32(a, qf[st], s[kb]);
            }
        }

        // ---- masking: keys >= key_end, and keys beyond the causal limit ----
        if (MASK) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (key >= key_end || key > lim) s[kb][r] = kNegInf;
                }
        }

        // ---- online softmax (row = this lane's query) ----
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = max_halves(mx);
        const float m_new = fmaxf(m_run, mx);
        // a row that has seen no allowed key yet keeps m = -inf; use 0 as its
        // reference so that no -inf - -inf is formed
        const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
        const float alpha = (m_run == kNegInf) ? 0.0f : fast_exp2((m_run - m_use) * c);
        const float mc = m_use * c;
        float lsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float pv = fast_exp2(fmaf(s[kb][r], c, -mc));
                if (MASK) pv = (s[kb][r] == kNegInf) ? 0.0f : pv;
                s[kb][r] = pv;
                lsum += pv;
            }
        l_run = fmaf(l_run, alpha, lsum);
        m_run = m_new;
        // rescale O only when some row's max moved
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        }

        // ---- P (bf16, from the S^T registers) as the B operand of O^T += V^T P^T ----
        bf16x8_t pb[PS];
#pragma unroll
        for (int ps = 0; ps < PS; ++ps) {
            const int kb = ps >> 1, t2 = ps & 1;
            u32x4_t w;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = pack_bf16(s[kb][8 * t2 + 2 * e], s[kb][8 * t2 + 2 * e + 1]);
            pb[ps] = __builtin_bit_cast(bf16x8_t, w);
        }
#pragma unroll
        for (int ps = 0; ps < PS; ++ps) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d = db * 32 + col;
                const int ch = 2 * ps + half;
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(
                    Vt + d * BN + ((ch ^ (d % VCH)) * 8));
                o[db] = mfma32(a, pb[ps], o[db]);
            }
        }
    }
};

// Write 4 consecutive head dims of one output row.
template <bool OUT_F32>
__device__ __forceinline__ void store4(void *o, long idx, float a, float b, float c, float d)
{
    if (OUT_F32) {
        float4 v = make_float4(a, b, c, d);
        *reinterpret_cast<float4 *>(static_cast<float *>(o) + idx) = v;
    } else {
        u32x2_t v = {pack_bf16(a, b), pack_bf16(c, d)};
        *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(o) + idx) = v;
    }
}

// ---------------------------------------------------------------------------
// Staging of one K/V tile: global -> registers -> LDS.
// K chunks go straight to Ks (swizzled); V chunks are transposed into Vt.
// NTHR threads; each holds NK 16-byte chunks of K and NK of V, where the V
// chunks are 4 consecutive keys x 8 head dims (so each transposed LDS write is
// 4 keys wide).
// ---------------------------------------------------------------------------
template <int D, int BN, int NTHR>
struct TileStager {
    static constexpr int KCH = D / 8;
    static constexpr int VCH = BN / 8;
    static constexpr int NK = BN * KCH / NTHR;       // chunks per thread per tensor
    static constexpr int KROWS = NTHR / KCH;          // K rows per pass
    static constexpr int VGROUPS = NTHR / KCH;        // 4-key groups per V pass
    static_assert(NK % 4 == 0 && NK >= 4, "stager needs groups of 4 keys");

    u32x4_t kst[NK], vst[NK];

    const uint16_t *kbase, *vbase;
    int kstride_bytes;  // bytes between consecutive keys
    int key_end;        // keys >= key_end read as zero

    __device__ __forceinline__ void bind(const uint16_t *kb, const uint16_t *vb, long kstride,
                                         int kend)
    {
        kbase = kb;
        vbase = vb;
        kstride_bytes = (int)(kstride * 2);
        key_end = kend;
    }

    // Buffer descriptor over `rows` key rows starting at key `row0`: rows
    // beyond key_end fall outside the descriptor's byte range and the hardware
    // returns zero for them (no branch per load).  Built from uniform values,
    // so it lives in scalar registers.
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t *base,
                                                                int row0) const
    {
        const int valid = key_end - row0;
        const int nbytes = valid > 0 ? (valid - 1) * kstride_bytes + D * 2 : 0;
        return __builtin_amdgcn_make_buffer_rsrc(
            (void *)(base + (long)row0 * (kstride_bytes / 2)), (short)0, nbytes, kBufferFlags);
    }

    // t: thread index, passed through an opaque copy so that the per-thread
    // offsets are recomputed here instead of being hoisted (and kept live)
    // across the whole loop.
    __device__ __forceinline__ void load(int key0, int t)
    {
        const int ch = t % KCH;
        const int vk = (t / KCH) * kstride_bytes + ch * 16;
        const int vv = 4 * (t / KCH) * kstride_bytes + ch * 16;
#pragma unroll
        for (int i = 0; i < NK; ++i)
            kst[i] = __builtin_amdgcn_raw_buffer_load_b128(rows_rsrc(kbase, key0 + i * KROWS), vk,
                                                           0, 0);
#pragma unroll
        for (int i = 0; i < NK; ++i)
            vst[i] = __builtin_amdgcn_raw_buffer_load_b128(
                rows_rsrc(vbase, key0 + 4 * VGROUPS * (i / 4) + (i % 4)), vv, 0, 0);
    }

    __device__ __forceinline__ void store(uint16_t *__restrict__ Ks, uint16_t *__restrict__ Vt,
                                          int t) const
    {
        const int ch = t % KCH;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int row = t / KCH + i * KROWS;
            *reinterpret_cast<u32x4_t *>(Ks + row * D + ((ch ^ (row % KCH)) * 8)) = kst[i];
        }
#pragma unroll
        for (int g4 = 0; g4 < NK / 4; ++g4) {
            const int key = 4 * VGROUPS * g4 + 4 * (t / KCH);
            const int p0 = vt_pos(key);  // 4-aligned, the 4 keys stay adjacent
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = ch * 8 + e;
                const int j = e >> 1;
                const u32x4_t *w = &vst[4 * g4];
                uint32_t lo, hi;
                if (e & 1) {
                    lo = (w[0][j] >> 16) | (w[1][j] & 0xffff0000u);
                    hi = (w[2][j] >> 16) | (w[3][j] & 0xffff0000u);
                } else {
                    lo = (w[0][j] & 0xffffu) | (w[1][j] << 16);
                    hi = (w[2][j] & 0xffffu) | (w[3][j] << 16);
                }
                *reinterpret_cast<u32x2_t *>(Vt + d * BN + (((p0 >> 3) ^ (d % VCH)) * 8) +
                                             (p0 & 7)) = u32x2_t{lo, hi};
            }
        }
    }
};

// An opaque copy of v: the compiler must assume it changes, so values derived
// from it are recomputed where they are used rather than hoisted out of loops.
__device__ __forceinline__ int opaque(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// Load this lane's Q fragment (B operand of S^T = K Q^T): head dims
// 16*st + 8*half .. +7 of one query row, for st = 0..D/16-1.  Rows outside
// the problem load as zero.  A negative scale is applied by negating Q here.
template <int D>
__device__ __forceinline__ void load_q(bf16x8_t (&qf)[D / 16], const uint16_t *qrow, bool valid,
                                       int half, uint32_t qflip)
{
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
        u32x4_t w = valid ? ld16(qrow + 16 * st + 8 * half) : u32x4_t{};
        w ^= qflip;
        qf[st] = __builtin_bit_cast(bf16x8_t, w);
    }
}

// ---------------------------------------------------------------------------
// Prefill: one workgroup = 4 waves = 128 query rows of one (b, hq); K/V tiles
// of BN keys stream through a double-buffered LDS stage.
// ---------------------------------------------------------------------------
template <int D>
struct PrefillTraits {
    static constexpr int BN = D == 64 ? 128 : 64;
};

template <int D, bool OUT_F32>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
fa_prefill_kernel(const Params p)
{
    constexpr int BM = kPrefillBM;
    constexpr int BN = PrefillTraits<D>::BN;
    constexpr int TILE = BN * D;
    using WT = WaveTile<D, BN>;
    using ST = TileStager<D, BN, 256>;

    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;

    const int BH = p.B * p.Hq;
    const int ND = p.domains;
    const int x = blockIdx.x % ND;           // scheduling domain (XCD)
    const int jw = blockIdx.x / ND;          // workgroup index inside the domain
    const int Gx = gridDim.x / ND;
    const int BHx = BH / ND;                 // (b, hq) pairs of this domain
    const int Nx = BHx * p.n_mblocks;        // items of this domain
    const long kstride = (long)p.Hkv * D;    // elements between consecutive keys

    for (int t = 0; t * Gx < Nx; ++t) {
        const int li = t * Gx + ((t & 1) ? (Gx - 1 - jw) : jw);
        if (li >= Nx) continue;
        const int rank = li / BHx;
        const int bh = (li % BHx) * ND + x;
        const int mb = p.causal ? (p.n_mblocks - 1 - rank) : rank;
        const int b = bh / p.Hq;
        const int hq = bh % p.Hq;
        const int g = hq / p.group;

        const int row0 = mb * BM;                       // first query row of the block
        const int wrow0 = row0 + wave * 32;             // first row of this wave
        const int qi = wrow0 + col;                     // this lane's query row
        const int last_row = min(row0 + BM, p.Sq) - 1;  // last valid row of the block
        const int wlast = min(wrow0 + 31, p.Sq - 1);    // last valid row of the wave

        int n_tiles = (p.Sk + BN - 1) / BN;
        if (p.causal) {
            const int hi = last_row + p.off;            // largest allowed key of the block
            n_tiles = hi < 0 ? 0 : min(n_tiles, hi / BN + 1);
        }

        bf16x8_t qf[D / 16];
        load_q<D>(qf, p.q + (((long)b * p.Sq + qi) * p.Hq + hq) * D, qi < p.Sq, half, p.qflip);

        const uint16_t *kbase = p.k + ((long)b * p.Sk * p.Hkv + g) * D;
        const uint16_t *vbase = p.v + ((long)b * p.Sk * p.Hkv + g) * D;

        f32x16_t o[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
        float m_run = kNegInf, l_run = 0.0f;

        ST stg;
        stg.bind(kbase, vbase, kstride, p.Sk);
        if (n_tiles > 0) {
            stg.load(0, opaque(tid));
            stg.store(lds, lds + TILE, opaque(tid));
        }
        __syncthreads();

        const int lim_lane = p.causal ? qi + p.off : 0x7fffffff;
        const int wmin_lim = p.causal ? wrow0 + p.off : 0x7fffffff;   // smallest limit of the wave
        const int wmax_lim = p.causal ? wlast + p.off : 0x7fffffff;   // largest limit of the wave

        for (int n = 0; n < n_tiles; ++n) {
            const int buf = n & 1;
            if (n + 1 < n_tiles) stg.load((n + 1) * BN, opaque(tid));

            const int key0 = n * BN;
            const uint16_t *Ks = lds + buf * 2 * TILE;
            const uint16_t *Vt = Ks + TILE;
            if (wrow0 < p.Sq && key0 <= wmax_lim) {   // tile not fully masked for this wave
                const bool need_mask = (key0 + BN > p.Sk) || (key0 + BN - 1 > wmin_lim);
                if (need_mask)
                    WT::template step<true>(Ks, Vt, qf, o, m_run, l_run, p.c, col, half, key0,
                                            p.Sk, lim_lane);
                else
                    WT::template step<false>(Ks, Vt, qf, o, m_run, l_run, p.c, col, half, key0,
                                             p.Sk, lim_lane);
            }

            if (n + 1 < n_tiles) {
                uint16_t *Kn = lds + (buf ^ 1) * 2 * TILE;
                stg.store(Kn, Kn + TILE, opaque(tid));
            }
            __syncthreads();
        }

        // ---- epilogue: O = O / l, LSE = ln(2) * (c * m + log2 l) ----
        const float l = add_halves(l_run);
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        if (qi < p.Sq) {
            const long obase = (((long)b * p.Sq + qi) * p.Hq + hq) * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int d0 = db * 32 + 8 * gq + 4 * half;
                    store4<OUT_F32>(p.o, obase + d0, o[db][4 * gq] * inv,
                                    o[db][4 * gq + 1] * inv, o[db][4 * gq + 2] * inv,
                                    o[db][4 * gq + 3] * inv);
                }
            if (p.lse && half == 0)
                p.lse[((long)b * p.Hq + hq) * p.Sq + qi] =
                    l > 0.0f ? (m_run * p.c + __log2f(l)) * kLn2 : kNegInf;
        }
    }
}

// ---------------------------------------------------------------------------
// Split-key decode: one wave per (b, KV head g, split).  Its 32 MFMA columns
// are the (query row, head-in-group) pairs of KV head g: column j is query
// j / group, head g * group + j % group; columns >= Sq * group are padding.
// ---------------------------------------------------------------------------
template <int D, bool OUT_F32>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
fa_decode_split_kernel(const Params p)
{
    constexpr int BN = kDecodeBN;
    constexpr int TILE = BN * D;
    using WT = WaveTile<D, BN>;
    using ST = TileStager<D, BN, 64>;

    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * TILE];

    const int lane = threadIdx.x;
    const int col = lane & 31;
    const int half = lane >> 5;

    const int item = blockIdx.x;
    const int s = item % p.num_splits;
    const int bg = item / p.num_splits;
    const int b = bg / p.Hkv;
    const int g = bg % p.Hkv;

    const int rows = p.Sq * p.group;
    const bool valid = col < rows;
    const int qi = valid ? col / p.group : 0;
    const int hq = g * p.group + (valid ? col % p.group : 0);

    const int k_begin = s * p.split_len;
    int k_end = min(k_begin + p.split_len, p.Sk);
    if (p.causal) k_end = min(k_end, p.Sq - 1 + p.off + 1);   // beyond every row's limit
    const int n_tiles = k_end > k_begin ? (k_end - k_begin + BN - 1) / BN : 0;

    bf16x8_t qf[D / 16];
    load_q<D>(qf, p.q + (((long)b * p.Sq + qi) * p.Hq + hq) * D, valid, half, p.qflip);

    const long kstride = (long)p.Hkv * D;
    const uint16_t *kbase = p.k + ((long)b * p.Sk * p.Hkv + g) * D;
    const uint16_t *vbase = p.v + ((long)b * p.Sk * p.Hkv + g) * D;

    f32x16_t o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
    float m_run = kNegInf, l_run = 0.0f;

    const int lim_lane = p.causal ? qi + p.off : 0x7fffffff;
    const int wmin_lim = p.causal ? p.off : 0x7fffffff;   // row 0 has the smallest limit

    ST stg;
    stg.bind(kbase, vbase, kstride, k_end);
    if (n_tiles > 0) stg.load(k_begin, opaque(lane));
    for (int n = 0; n < n_tiles; ++n) {
        const int key0 = k_begin + n * BN;
        __syncthreads();                      // previous tile's LDS reads are done
        stg.store(lds, lds + TILE, opaque(lane));
        __syncthreads();
        if (n + 1 < n_tiles) stg.load(key0 + BN, opaque(lane));
        const bool need_mask = (key0 + BN > k_end) || (key0 + BN - 1 > wmin_lim);
        // keys are counted relative to the tile inside step(); pass absolute bounds
        if (need_mask)
            WT::template step<true>(lds, lds + TILE, qf, o, m_run, l_run, p.c, col, half, key0,
                                    k_end, lim_lane);
        else
            WT::template step<false>(lds, lds + TILE, qf, o, m_run, l_run, p.c, col, half, key0,
                                     k_end, lim_lane);
    }

    const float l = add_halves(l_run);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float lse = l > 0.0f ? (m_run * p.c + __log2f(l)) * kLn2 : kNegInf;
    if (!valid) return;
    if (p.num_splits == 1) {
        const long obase = (((long)b * p.Sq + qi) * p.Hq + hq) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d0 = db * 32 + 8 * gq + 4 * half;
                store4<OUT_F32>(p.o, obase + d0, o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv,
                                o[db][4 * gq + 2] * inv, o[db][4 * gq + 3] * inv);
            }
        if (p.lse && half == 0) p.lse[((long)b * p.Hq + hq) * p.Sq + qi] = lse;
    } else {
        const long prow = (((long)s * p.B + b) * p.Hq + hq) * p.Sq + qi;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d0 = db * 32 + 8 * gq + 4 * half;
                store4<true>(p.part_o, prow * D + d0, o[db][4 * gq] * inv,
                             o[db][4 * gq + 1] * inv, o[db][4 * gq + 2] * inv,
                             o[db][4 * gq + 3] * inv);
            }
        if (half == 0) p.part_lse[prow] = lse;
    }
}

// ---------------------------------------------------------------------------
// Merge of split partials, one wave per output row (b, hq, i):
//   M = max_s LSE_s, w_s = exp(LSE_s - M), LSE = M + ln sum_s w_s,
//   O = sum_s w_s O_s / sum_s w_s; splits with LSE_s = -inf weigh 0, and a row
//   whose splits are all -inf gets O = 0, LSE = -inf.
// ---------------------------------------------------------------------------
template <int D, bool OUT_F32>
__global__ void __launch_bounds__(64) fa_merge_kernel(const Params p)
{
    const int lane = threadIdx.x;
    const long row = blockIdx.x;                 // (b, hq, i) with i fastest
    const long n_rows = (long)p.B * p.Hq * p.Sq;
    const int ns = p.num_splits;

    float M = kNegInf;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, p.part_lse[s * n_rows + row]);
    const float Mu = (M == kNegInf) ? 0.0f : M;

    constexpr int PER = D / 64;                  // head dims per lane
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
    float wsum = 0.0f;
    for (int s = 0; s < ns; ++s) {
        const float ls = p.part_lse[s * n_rows + row];
        const float w = (ls == kNegInf) ? 0.0f : __expf(ls - Mu);
        wsum += w;
        const float *po = p.part_o + (s * n_rows + row) * D + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, po[e], acc[e]);
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;

    const int i = (int)(row % p.Sq);
    const int hq = (int)((row / p.Sq) % p.Hq);
    const int b = (int)(row / ((long)p.Sq * p.Hq));
    const long obase = (((long)b * p.Sq + i) * p.Hq + hq) * D + lane * PER;
    if (OUT_F32) {
#pragma unroll
        for (int e = 0; e < PER; ++e) static_cast<float *>(p.o)[obase + e] = acc[e] * inv;
    } else {
        if (PER == 2) {
            *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(p.o) + obase) =
                pack_bf16(acc[0] * inv, acc[PER - 1] * inv);
        } else {
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                __bf16 h = (__bf16)(acc[e] * inv);
                static_cast<uint16_t *>(p.o)[obase + e] = __builtin_bit_cast(uint16_t, h);
            }
        }
    }
    if (p.lse && lane == 0)
        p.lse[row] = wsum > 0.0f ? Mu + __logf(wsum) : kNegInf;
}

Params make_params(const Launch &L)
{
    Params p;
    p.q = static_cast<const uint16_t *>(L.q);
    p.k = static_cast<const uint16_t *>(L.k);
    p.v = static_cast<const uint16_t *>(L.v);
    p.o = L.o;
    p.lse = L.lse;
    p.part_o = L.part_o;
    p.part_lse = L.part_lse;
    p.B = L.B;
    p.Hq = L.Hq;
    p.Hkv = L.Hkv;
    p.Sq = L.Sq;
    p.Sk = L.Sk;
    p.group = L.Hq / L.Hkv;
    p.causal = L.causal;
    p.off = L.Sk - L.Sq;
    const float log2e = 1.4426950408889634f;
    p.c = (L.scale < 0.0f ? -L.scale : L.scale) * log2e;
    p.qflip = L.scale < 0.0f ? 0x80008000u : 0u;
    p.n_mblocks = (L.Sq + kPrefillBM - 1) / kPrefillBM;
    p.domains = 1;
    p.num_splits = L.num_splits;
    p.split_len = L.split_len;
    return p;
}

}  // namespace

hipError_t launch_prefill(const Launch &L)
{
    Params p = make_params(L);
    const int BH = L.B * L.Hq;
    const int grid = L.grid;
    // one XCD domain per (b, hq) residue class when both counts divide by 8
    p.domains = (BH % 8 == 0 && grid % 8 == 0) ? 8 : 1;
    dim3 g(grid), blk(256);
    if (L.D == 128) {
        if (L.o_f32)
            hipLaunchKernelGGL((fa_prefill_kernel<128, true>), g, blk, 0, L.stream, p);
        else
            hipLaunchKernelGGL((fa_prefill_kernel<128, false>), g, blk, 0, L.stream, p);
    } else {
        if (L.o_f32)
            hipLaunchKernelGGL((fa_prefill_kernel<64, true>), g, blk, 0, L.stream, p);
        else
            hipLaunchKernelGGL((fa_prefill_kernel<64, false>), g, blk, 0, L.stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_decode(const Launch &L)
{
    Params p = make_params(L);
    dim3 g(L.B * L.Hkv * L.num_splits), blk(64);
    if (L.D == 128) {
        if (L.o_f32)
            hipLaunchKernelGGL((fa_decode_split_kernel<128, true>), g, blk, 0, L.stream, p);
        else
            hipLaunchKernelGGL((fa_decode_split_kernel<128, false>), g, blk, 0, L.stream, p);
    } else {
        if (L.o_f32)
            hipLaunchKernelGGL((fa_decode_split_kernel<64, true>), g, blk, 0, L.stream, p);
        else
            hipLaunchKernelGGL((fa_decode_split_kernel<64, false>), g, blk, 0, L.stream, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || L.num_splits == 1) return e;
    dim3 gm((unsigned)((long)L.B * L.Hq * L.Sq));
    if (L.D == 128) {
        if (L.o_f32)
            hipLaunchKernelGGL((fa_merge_kernel<128, true>), gm, blk, 0, L.stream, p);
        else
            hipLaunchKernelGGL((fa_merge_kernel<128, false>), gm, blk, 0, L.stream, p);
    } else {
        if (L.o_f32)
            hipLaunchKernelGGL((fa_merge_kernel<64, true>), gm, blk, 0, L.stream, p);
        else
            hipLaunchKernelGGL((fa_merge_kernel<64, false>), gm, blk, 0, L.stream, p);
    }
    return hipGetLastError();
}

}  // namespace fa
