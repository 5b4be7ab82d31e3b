// fa_kernels.hip -- fused attention forward kernels for gfx950 (CDNA4, wave64).
//
// What is computed: O = softmax(scale * Q K^T [causal]) V and LSE per query
// row, never writing S or P to HBM.  The structure follows the FlashAttention
// forward main loop laid out in "SM80 内核实现对比" (Inference Cookbook): Q kept
// in registers for the whole key loop (section 5.3, Q_in_regs), K/V tiles
// staged through on-chip memory by asynchronous 16-byte copies with zero fill
// at the edges (sections 2.1 and 4.1; the pages' pipeline is two stages deep,
// the rings here three), the S = Q K^T product,
// the online softmax, then P V with P taken from registers (section 5.2), and
// an XOR-swizzled on-chip layout (section 6.3).  The online-softmax pieces --
// row max, exp, row sum, rescale, causal mask -- are those named in
// "从 Volta/Turing、Ampere、Ada 到 Hopper：硬件、PTX 与 Kernel 编程范式演进",
// section "Attention 的瓶颈会在 Tensor Core 与 CUDA Core 之间迁移".
//
// What is CDNA4-specific (and differs from the pages' SM80/SM90 designs):
//  * Both products run on v_mfma_f32_32x32x16_bf16 in the transposed form
//    S^T = K Q^T and O^T = V^T P^T.  In the 32x32 accumulator layout a lane owns
//    one output column (here: one query) and 16 rows (keys, or head dims), so
//    the row max and row sum need a single cross-lane step (v_permlane32_swap)
//    and the per-query rescale factor is lane-local.
//  * P never leaves registers: the S^T accumulator registers, converted to
//    bf16, are the B operand of the PV MFMA.  The A operand V^T is read from
//    the natural [key][d] V tile with the transposing LDS read
//    ds_read_b64_tr_b16 (each lane gets 4 consecutive keys of one head dim),
//    so V needs no transposed copy anywhere.
//  * K and V tiles go from HBM to LDS with buffer_load_dwordx4 ... lds (no
//    staging registers); the buffer descriptor's byte range makes rows past
//    the last key read as zero.
//  * The LDS swizzle (chunk ^ swz(row)) is chosen so that both the 32-row
//    ds_read_b128 of K and the 4-row x 64-byte transposing read of V hit
//    distinct banks, for a 32- and a 64-bank LDS alike.
//  * The running max is a lazy reference: it only moves when a row's max
//    grows by more than 2^8 in exp2 units, so the O rescale is skipped on
//    almost every tile.  P values then stay below 2^8, which bf16 and the fp32
//    accumulators hold without loss; the result is the same function.
//  * Prefill runs a persistent grid (one workgroup per CU) that walks
//    (batch, head, query block) items in a snake order that balances the
//    causal lengths, and keeps all blocks of a head on one XCD so that their
//    K/V re-reads hit that XCD's L2.  Two kernels: 32 query rows per wave and
//    two waves per SIMD (the default), or 64 rows per wave and one wave per
//    SIMD with a hand-pipelined block loop (half the LDS reads per flop).
//  * The HBM -> LDS copies are issued as inline asm so that the compiler does
//    not make LDS reads wait for copies still in flight (see lds_dma16_pair).
//  * Decode (few query rows per KV head) runs a split-key kernel, one wave per
//    (batch, KV head, key range) with a three-tile LDS ring, which writes
//    partial (O_s, LSE_s); a merge pass combines them with log-sum-exp weights.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "fa_launch.h"

namespace fa {
namespace kern {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((__vector_size__(64)));
typedef float f32x4_t __attribute__((__vector_size__(16)));
typedef uint32_t u32x4_t __attribute__((__vector_size__(16)));
typedef uint32_t u32x2_t __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegInf = -__builtin_inff();
// Word 3 of a gfx9-family buffer descriptor: 32-bit data format, so that
// untyped dword loads are valid; out-of-range offsets return zero.
constexpr int kBufferFlags = 0x00020000;
// The lazy running max moves when a row max exceeds it by more than this
// (exp2 units): P stays below 2^8.
constexpr float kRescaleThreshold = 8.0f;
#ifndef FA_USE_PRIO
#define FA_USE_PRIO 1
#endif
constexpr bool kUsePrio = FA_USE_PRIO;

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
    int head_major;   // prefill: walk a domain's items head by head (else rank by rank)
    int num_splits, split_len;
};

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// S^T MFMAs of the hand-ordered loops (the 64-row prefill's fast block, the
// dK/dV pipeline), with the accumulator in VGPRs.  The VALU reads S next,
// and the compiler keeps every accumulator of those kernels in AGPRs (moving
// S out would cost 32 v_accvgpr_read per block), so these two are written
// out; the B operand (Q, or the K / V rows) comes straight from AGPRs.  The compiler does not see
// the MFMA inside, so it would also not wait for its result: the chain of
// one accumulator ends in mfma_s_drain, which takes the accumulators as
// operands, so nothing the compiler emits can touch them before the wait.
// (It could still copy or spill one between the MFMA and the drain; the
// build scans the generated code for any such access and rejects it.)
__device__ __forceinline__ void mfma_s_first(f32x16_t &d, bf16x8_t a, bf16x8_t b)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_s_next(f32x16_t &d, bf16x8_t a, bf16x8_t b)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}

// The wait after the last S MFMAs of a block (24 wait states; the 8-pass
// MFMA needs about half of that), before anything may read or move S.
__device__ __forceinline__ void mfma_s_drain(f32x16_t &a, f32x16_t &b)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b)::"memory");
}
__device__ __forceinline__ void mfma_s_drain(f32x16_t &a)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a)::"memory");
}

// The same fence without the wait, for the end of the hand-ordered fast
// block: there the last S MFMAs are followed by the block's last P V and
// row-sum MFMAs and a quarter step of softmax work (16 or more instructions,
// in an order fixed by scheduling fences), which already cover the 8-pass
// MFMA's result latency.  The build's scan of the generated code checks that
// enough wait states pass before any access to S (asm_check.py); the drain
// cost about 90 cycles per 32-key block.
__device__ __forceinline__ void mfma_s_fence(f32x16_t &a, f32x16_t &b)
{
    asm volatile("" : "+v"(a), "+v"(b)::"memory");
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

// Two floats to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// The two bf16 halves of a packed word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ u32x4_t ld16(const uint16_t *p)
{
    return *reinterpret_cast<const u32x4_t *>(p);
}

// Wave issue priority (s_setprio): a wave raises it while it issues an MFMA
// chain, so that with two waves on a SIMD the matrix pipe is fed first and the
// other wave's VALU work fills the cycles in between.
template <int P, bool ON = true>
__device__ __forceinline__ void set_prio()
{
    if (kUsePrio && ON) __builtin_amdgcn_s_setprio(P);
}

// Wait until this wave's outstanding vector-memory operations (including the
// HBM -> LDS copies) are done.  gfx9 s_waitcnt: vmcnt(0), expcnt(7), lgkmcnt(15).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Pins the computation of a VGPR value before this point (an empty volatile
// asm that reads it), so that a software-pipelined step keeps its share of
// the VALU work between its own MFMAs.
__device__ __forceinline__ void keep(uint32_t a) { asm volatile("" ::"v"(a)); }
__device__ __forceinline__ void keep(float a) { asm volatile("" ::"v"(a)); }

// Workgroup barrier between phases, without the memory fence of
// __syncthreads (which would wait for the K/V copies still in flight).  The
// empty asm statements keep the compiler from moving LDS accesses across it,
// the scheduling fences any other instruction: without them the scheduler
// hoisted a V phase's register-only softmax work above the barrier into the
// M phase, where it defeats the alternation.
__device__ __forceinline__ void pp_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// LDS tile layout, K and V alike: [rows][D] bf16, rows of 2*D bytes; the
// 16-byte chunk c of row r sits at chunk c ^ swz(r).  Bits ri of the row:
//   D = 128 (16 chunks): swz = r0<<3 | r1<<2 | (r0^r2)<<1 | (r2^r3)
//   D =  64 ( 8 chunks): swz = r1<<2 | (r0^r2)<<1 | (r0^r3)
//   D = 256 (32 chunks): as D = 128.  A row is 512 bytes, twice the 64 banks'
//     width, so a chunk's bank depends on its index mod 16 only, which the
//     D = 128 pattern already permutes conflict-free.
// Any 16 consecutive rows at one chunk (the K read) and any 4 rows starting at
// a multiple of 4 over an aligned block of 4 chunks (the V transposing read)
// land on distinct banks.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz(int r)
{
    const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
    if (D >= 128) return (r0 << 3) | (r1 << 2) | ((r0 ^ r2) << 1) | (r2 ^ r3);
    return (r1 << 2) | ((r0 ^ r2) << 1) | (r0 ^ r3);
}

// The swizzle of the FP8 tiles (rows of 128 bytes, eight 16-byte chunks).
// Their V^T read (ds_read_b64_tr_b8) takes 8 bytes per lane from the rows
// {a..a+3, a+8..a+11}, a = 0 or 4 mod 16, 32 bytes per row; with 64 banks
// (32 lanes of 8 bytes per cycle) the even rows of that set, and the odd
// ones, need distinct 32-byte positions: distinct swz >> 1.  swz<64> above
// maps rows a and a+8 to the same position (a 2-way conflict the SQ counters
// showed, 8.5 M conflict cycles per call); this one keeps that apart, the
// K reads' conditions (distinct over 8 consecutive rows, and over the even
// and the odd rows of 16) and the 32-bank ones, checked by simulation of
// every read of the FP8 kernel.
__device__ __forceinline__ int swz_fp8(int r) { return (r & 7) ^ (5 * ((r >> 3) & 1)); }

// Race checks of the LDS rings, in debug builds of the library only
// (FA_LDS_CHECK = 0 in the product build).  A ring stage must be ready (its
// copies landed and every wave past the barrier that follows the wait) before
// it is read, and reusable (every wave done reading it) before the copies of
// a later tile go into it ("理解 H100：从硬件数据路径到 Nsight Compute 瓶颈分析",
// section 6, the asynchronous pipeline's stage states).
//  * FA_LDS_CHECK = 1 (synchronous copies): each copy is waited for
//    (vmcnt(0)) right after it is issued, so every stage is ready long
//    before the kernel's own wait and barrier would make it so.  A missing or
//    too-short wait in the normal build then shows as a bitwise difference.
//  * FA_LDS_CHECK = 2 (poison): before each copy, the issuing lane writes
//    all-ones -- NaN as bf16, fp32 and E4M3 -- into the LDS bytes that copy
//    will fill, and waits for the write.  A wave still reading the stage
//    (not reusable), or reading it before the copy lands (not ready), takes
//    the poison instead of data it could have silently got away with.
#ifndef FA_LDS_CHECK
#define FA_LDS_CHECK 0
#endif

template <int BYTES>
__device__ __forceinline__ void lds_check_before_copy(char *dst)
{
#if FA_LDS_CHECK == 2
    const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    char __attribute__((address_space(3))) *d =
        (char __attribute__((address_space(3))) *)(lds_void_t *)dst + lane * BYTES;
    if constexpr (BYTES == 16)
        *(u32x4_t __attribute__((address_space(3))) *)d = (u32x4_t){~0u, ~0u, ~0u, ~0u};
    else
        *(uint32_t __attribute__((address_space(3))) *)d = ~0u;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#else
    (void)dst;
#endif
}

__device__ __forceinline__ void lds_check_after_copy()
{
#if FA_LDS_CHECK == 1
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#endif
}

// One HBM -> LDS copy instruction: buffer_load_dwordx4 ... lds writes the 64
// lanes' 16 bytes at consecutive LDS addresses from M0 on.  It is issued as
// inline asm on purpose: the compiler tracks its own LDS-DMA loads and, unable
// to prove that a later transposing LDS read does not touch the destination,
// waits for every copy in flight (vmcnt(0)) before that read -- which would
// expose the full HBM latency of the tiles prefetched ahead.  The kernels wait
// for the copies themselves (wait_vmem / wait_tiles_ahead, then a barrier).
// M0 is saved and restored around the copies (the compiler reserves it).
//
// lds_dma16_pair issues the K and the V copy of one lane chunk: same
// offsets, two descriptors, two LDS destinations.  STREAM marks them
// non-temporal: data read once (the decode's K/V) then does not displace
// cache lines that are still needed, such as output another kernel left
// dirty, whose write-back would otherwise be charged to the streaming read.
template <bool STREAM = false>
__device__ __forceinline__ void lds_dma16_pair(char *lds_k, char *lds_v, int voff, u32x4_t kd,
                                               u32x4_t vd)
{
    const uint32_t m0k = (uint32_t)reinterpret_cast<uintptr_t>((lds_void_t *)lds_k);
    const uint32_t m0v = (uint32_t)reinterpret_cast<uintptr_t>((lds_void_t *)lds_v);
    uint32_t saved;
    lds_check_before_copy<16>(lds_k);
    lds_check_before_copy<16>(lds_v);
    if (STREAM)
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %3, %4, 0 offen nt lds\n\t"
            "s_mov_b32 m0, %2\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %3, %5, 0 offen nt lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0k), "s"(m0v), "v"(voff), "s"(kd), "s"(vd)
            : "memory");
    else
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %3, %4, 0 offen lds\n\t"
            "s_mov_b32 m0, %2\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %3, %5, 0 offen lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0k), "s"(m0v), "v"(voff), "s"(kd), "s"(vd)
            : "memory");
    lds_check_after_copy();
}

// One copy of lds_dma16_pair's kind into one destination.
template <bool STREAM = false>
__device__ __forceinline__ void lds_dma16(char *lds, int voff, u32x4_t d)
{
    const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void_t *)lds);
    uint32_t saved;
    lds_check_before_copy<16>(lds);
    if (STREAM)
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0), "v"(voff), "s"(d)
            : "memory");
    else
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0), "v"(voff), "s"(d)
            : "memory");
    lds_check_after_copy();
}

// HBM -> LDS copy of one K and one V tile of BN keys by NW waves.  One
// buffer_load_dwordx4 ... lds instruction writes 1 KiB: 64 lanes x 16 bytes at
// consecutive LDS addresses.  Lane l of instruction q fills tile row
// q * RPI + l / CPR at physical chunk l % CPR, i.e. it loads the logical chunk
// (l % CPR) ^ swz(row) of that key's row.
template <int D, int BN, int NW, bool STREAM = false, bool FP8SWZ = false>
struct TileLoader {
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row
    static constexpr int RPI = 64 / CPR;              // rows per instruction
    static constexpr int NQ = BN / RPI;               // instructions per tensor
    static constexpr int PER_WAVE = NQ / NW;
    static constexpr int TILE_BYTES = BN * D * 2;
    static_assert(NQ % NW == 0, "instructions must split evenly over the waves");

    u32x4_t kdesc, vdesc;   // K and V rows [0, key_end) of one (batch, KV head)

    __device__ __forceinline__ static int row_swz(int row)
    {
        return FP8SWZ ? swz_fp8(row) : swz<D>(row);
    }
    int kstride_bytes;      // bytes between consecutive keys in HBM

    // Descriptors whose byte range ends with row key_end - 1, so that rows
    // at or beyond key_end read as zero.  Uniform values only (scalar
    // registers).  Words: base address bits 31:0; bits 47:32 (stride 0);
    // byte range; flags.  Byte offsets stay below 2^31: the host checks
    // that K and V of one batch are under 2 GiB.
    __device__ __forceinline__ void setup(const uint16_t *kbase, const uint16_t *vbase,
                                          int kstride, int key_end)
    {
        kstride_bytes = kstride;
        const uint32_t nbytes = key_end > 0 ? (uint32_t)((key_end - 1) * kstride + D * 2) : 0u;
        const uint64_t ka = reinterpret_cast<uint64_t>(kbase);
        const uint64_t va = reinterpret_cast<uint64_t>(vbase);
        kdesc = (u32x4_t){(uint32_t)ka, (uint32_t)(ka >> 32) & 0xffffu, nbytes,
                          (uint32_t)kBufferFlags};
        vdesc = (u32x4_t){(uint32_t)va, (uint32_t)(va >> 32) & 0xffffu, nbytes,
                          (uint32_t)kBufferFlags};
    }

    // Issue the copies of keys [key0, key0 + BN) into the K and V tiles at
    // lds_k / lds_v.  key0 is a multiple of 16.
    __device__ __forceinline__ void issue(char *lds_k, char *lds_v, int key0, int wave,
                                          int lane) const
    {
        const int toff = key0 * kstride_bytes;   // uniform
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int q = i * NW + wave;
            const int row = q * RPI + lane / CPR;          // tile-relative row
            const int voff = toff + row * kstride_bytes + (((lane % CPR) ^ row_swz(row)) * 16);
            lds_dma16_pair<STREAM>(lds_k + q * 1024, lds_v + q * 1024, voff, kdesc, vdesc);
        }
    }

    // The copies of one tensor only (V if IS_V, else K).
    template <bool IS_V>
    __device__ __forceinline__ void issue_one(char *dst, int key0, int wave, int lane) const
    {
        const int toff = key0 * kstride_bytes;
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int q = i * NW + wave;
            const int row = q * RPI + lane / CPR;
            const int voff = toff + row * kstride_bytes + (((lane % CPR) ^ row_swz(row)) * 16);
            lds_dma16<STREAM>(dst + q * 1024, voff, IS_V ? vdesc : kdesc);
        }
    }
};

// The same copies out of a paged K/V cache: [pages][page_size][Hkv][D], with
// one sequence's logical page p stored in cache page table[p].  page_size is
// a power of two >= 16: a BN-key tile (BN = 32, starting at a multiple of 32)
// lies in one page (PPT = 1, page_size >= BN) or covers PPT = BN / page_size
// whole pages, each holding NQ / PPT of the tile's copy instructions.
//
// The page ids of the split's pages are loaded once per wave into VGPRs (lane
// l of register r holds page p_first + 64 r + l) and read back with
// v_readlane: no memory access in the key loop besides the copies, whose
// vmcnt bookkeeping the ring relies on.  A page id outside [0, num_pages) and
// rows at or beyond key_end get an empty byte range: they read as zeros, so a
// bad table entry can give wrong numbers but no out-of-bounds access.
template <int D, int BN, int PPT>
struct PagedTileLoader {
    static constexpr int CPR = D / 8;
    static constexpr int RPI = 64 / CPR;
    static constexpr int NQ = BN / RPI;
    static constexpr int PER_WAVE = NQ;                // one wave per ring
    static constexpr int TILE_BYTES = BN * D * 2;
    static constexpr int R = kPagedIdRegs;
    static_assert(PPT >= 1 && NQ % PPT == 0, "a page must hold whole copy instructions");

    int pid[R];              // per lane: page ids of the split's pages
    const uint16_t *kc, *vc; // caches, already offset to the KV head
    long page_elems;         // elements per cache page (page_size * Hkv * D)
    int p_first;             // first logical page of the split
    int shift;               // log2(page_size)
    int num_pages;
    int key_end;             // keys at or beyond read as zero
    int kstride_bytes;       // bytes between consecutive keys of a page

    // Issue the page-id loads (vector loads; the first issue() waits for
    // them).  table: the sequence's block-table row.  Keys [k_begin, k_end).
    __device__ __forceinline__ void setup(const uint16_t *kcache, const uint16_t *vcache,
                                          const int *table, int max_pages, int k_begin, int k_end,
                                          int lg_page, int n_pages, long page_el, int kstride,
                                          int lane)
    {
        kc = kcache;
        vc = vcache;
        page_elems = page_el;
        shift = lg_page;
        num_pages = n_pages;
        key_end = k_end;
        kstride_bytes = kstride;
        p_first = k_begin >> lg_page;
        // unconditional loads (no branch around them), clamped into the
        // row: entries past the split's last page are loaded but never used
        const int p_last = min(k_end > k_begin ? (k_end - 1) >> lg_page : p_first, max_pages - 1);
#pragma unroll
        for (int r = 0; r < R; ++r)
            pid[r] = table[max(min(p_first + 64 * r + lane, p_last), 0)];
    }

    // One descriptor per page the tile touches (PPT of them: the tile's NQ
    // copy instructions split evenly), based at that page.
    __device__ __forceinline__ void issue(char *lds_k, char *lds_v, int key0, int, int lane) const
    {
        issue_sel<0>(lds_k, lds_v, key0, lane);
    }
    // The copies of one tensor only (V if IS_V, else K) into dst.
    template <bool IS_V>
    __device__ __forceinline__ void issue_one(char *dst, int key0, int, int lane) const
    {
        issue_sel<IS_V ? 2 : 1>(dst, dst, key0, lane);
    }
    // WHICH: 0 both tensors, 1 K only (into lds_k), 2 V only (into lds_v)
    template <int WHICH>
    __device__ __forceinline__ void issue_sel(char *lds_k, char *lds_v, int key0, int lane) const
    {
        constexpr int QPP = NQ / PPT;                       // instructions per page
#pragma unroll
        for (int c = 0; c < PPT; ++c) {
            const int r0 = key0 + c * QPP * RPI;            // uniform: first key of the page chunk
            const int pg = r0 >> shift;
            const int rel = pg - p_first;
            // every register read back, then a scalar select: selecting the
            // register first becomes a dynamically indexed array in scratch
            int page = __builtin_amdgcn_readlane(pid[0], rel & 63);
#pragma unroll
            for (int r = 1; r < R; ++r) {
                const int cand = __builtin_amdgcn_readlane(pid[r], rel & 63);
                page = (rel >> 6) == r ? cand : page;
            }
            const int first = pg << shift;
            const int rows = min(key_end - first, 1 << shift);
            const bool ok = (unsigned)page < (unsigned)num_pages && rows > 0;
            page = ok ? page : 0;
            const uint32_t nbytes = ok ? (uint32_t)((rows - 1) * kstride_bytes + D * 2) : 0u;
            const uint64_t ka = reinterpret_cast<uint64_t>(kc + page * page_elems);
            const uint64_t va = reinterpret_cast<uint64_t>(vc + page * page_elems);
            const u32x4_t kd = {(uint32_t)ka, (uint32_t)(ka >> 32) & 0xffffu, nbytes,
                                (uint32_t)kBufferFlags};
            const u32x4_t vd = {(uint32_t)va, (uint32_t)(va >> 32) & 0xffffu, nbytes,
                                (uint32_t)kBufferFlags};
            const int base = (key0 - first + lane / CPR) * kstride_bytes;
#pragma unroll
            for (int i = 0; i < QPP; ++i) {
                const int q = c * QPP + i;
                const int row = q * RPI + lane / CPR;       // tile-relative row
                const int voff = base + q * RPI * kstride_bytes +
                                 (((lane % CPR) ^ swz<D>(row)) * 16);
                if (WHICH == 0)
                    lds_dma16_pair<true>(lds_k + q * 1024, lds_v + q * 1024, voff, kd, vd);
                else if (WHICH == 1)
                    lds_dma16<true>(lds_k + q * 1024, voff, kd);
                else
                    lds_dma16<true>(lds_v + q * 1024, voff, vd);
            }
        }
    }
};

// Per-lane LDS byte offsets (relative to a tile) of the operand reads.
//   K (A operand of S^T = K Q^T): lane (col, half) at k-step st reads the 16
//     bytes of head dims 16*st + 8*half .. +7 of key kb*32 + col.
//   V^T (A operand of O^T = V^T P^T) through ds_read_b64_tr_b16: in each
//     16-lane group, source lane 4j + s supplies 4 consecutive head dims of
//     key row k0 + j; the instruction hands lane 4s + e element e of those
//     four rows, i.e. 4 consecutive keys of one head dim.
template <int D>
//   The swizzle permutes chunk indices mod 16 only, so at D = 256 the second
//   256 bytes of a row repeat the first half's offsets + 256: only the first
//   16 chunks' offsets are kept in registers (kofs / vofs add the rest as an
//   immediate).
struct OperandOffsets {
    static constexpr int QS = D / 16;
    static constexpr int DB = D / 32;
    static constexpr int NK = QS < 8 ? QS : 8;     // k-steps within the first 256 bytes
    static constexpr int NV = DB < 4 ? DB : 4;     // d blocks within the first 256 bytes
    int k[NK];           // + kb * 32 rows
    int v[NV][2];        // [d block][second group of 4 keys]; + ps * 16 rows

    __device__ __forceinline__ int kofs(int st) const
    {
        if constexpr (NK == QS) return k[st];
        else return k[st % NK] + (st / NK) * 256;
    }
    __device__ __forceinline__ int vofs(int db, int sec) const
    {
        if constexpr (NV == DB) return v[db][sec];
        else return v[db % NV][sec] + (db / NV) * 256;
    }

    __device__ __forceinline__ void init(int lane)
    {
        const int col = lane & 31, half = lane >> 5;
#pragma unroll
        for (int st = 0; st < NK; ++st)
            k[st] = col * (2 * D) + (((2 * st + half) ^ swz<D>(col)) * 16);
        const int li = lane & 15, g = (lane >> 4) & 1;
#pragma unroll
        for (int db = 0; db < NV; ++db)
#pragma unroll
            for (int sec = 0; sec < 2; ++sec) {
                const int row = 4 * half + (li >> 2) + 8 * sec;
                const int d = db * 32 + 16 * g + 4 * (li & 3);
                v[db][sec] = row * (2 * D) + (((d >> 3) ^ swz<D>(row)) * 16) + (d & 7) * 2;
            }
    }
};

// ---------------------------------------------------------------------------
// One wave's share of a K/V tile held in LDS: S^T, online softmax, O^T += V^T P^T.
// Lane (col, half): query column `col`; after the S^T MFMA its register r of
// key block kb holds key kb*32 + 8*(r/4) + 4*half + (r%4).
// ---------------------------------------------------------------------------
template <int D, int BN>
struct WaveTile {
    static constexpr int QS = D / 16;
    static constexpr int KB = BN / 32;
    static constexpr int DB = D / 32;
    static constexpr int PS = BN / 16;

    template <bool MASK>
    __device__ __forceinline__ static void step(const char *__restrict__ Ks,
                                                const char *__restrict__ Vs,
                                                const OperandOffsets<D> &off,
                                                const bf16x8_t (&qf)[QS], f32x16_t (&o)[DB],
                                                float &m_ref, float &l_run, float &l_rnd, float c,
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
                const bf16x8_t a =
                    *reinterpret_cast<const bf16x8_t *>(Ks + off.kofs(st) + kb * 32 * 2 * D);
                s[kb] = mfma32(a, qf[st], s[kb]);
            }
        }

        // ---- masking: keys >= key_end, and keys beyond the causal limit ----
        if (MASK) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                // offsets 8*(r/4) + r%4 stay immediates (see BlockOps::mask)
                const int last = min(lim, key_end - 1) - (key0 + kb * 32 + 4 * half);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[kb][r] = (8 * (r >> 2) + (r & 3) > last) ? kNegInf : s[kb][r];
            }
        }

        // ---- online softmax (row = this lane's query) with a lazy reference max ----
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = max_halves(mx);
        // a row moves its reference when its max grew past the threshold (the
        // first allowed key always does: m_ref starts at -inf)
        const bool grow = (mx - m_ref) * c > kRescaleThreshold;
        if (__any(grow)) {
            const float m_new = grow ? mx : m_ref;
            const float alpha = (m_ref == kNegInf) ? 0.0f : fast_exp2((m_ref - m_new) * c);
            l_run *= alpha;
            l_rnd *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
            m_ref = m_new;
        }
        // rows that have not seen an allowed key keep m_ref = -inf; 0 stands in
        const float mc = (m_ref == kNegInf) ? 0.0f : m_ref * c;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float pv = fast_exp2(fmaf(s[kb][r], c, -mc));
                if (MASK) pv = (s[kb][r] == kNegInf) ? 0.0f : pv;
                s[kb][r] = pv;
                l_run += pv;
            }

        // ---- P (bf16, from the S^T registers) as the B operand of O^T += V^T P^T ----
        // PV step ps covers keys 16*ps .. +15; B element e of lane half h is key
        // 16*ps + 8*(e/4) + 4*h + e%4, which the two transposing reads of V
        // (keys 16*ps + 4*h + 0..3 and 16*ps + 8 + 4*h + 0..3) match.
#pragma unroll
        for (int ps = 0; ps < PS; ++ps) {
            const int kb = ps >> 1, t2 = ps & 1;
            u32x4_t w;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = pack_bf16(s[kb][8 * t2 + 2 * e], s[kb][8 * t2 + 2 * e + 1]);
            // l_rnd adds the rounded values that P V multiplies (normalises O);
            // l_run above the exact ones (feeds the LSE)
#pragma unroll
            for (int e = 0; e < 4; ++e) l_rnd += bf16_lo(w[e]) + bf16_hi(w[e]);
            const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4_t *)(Vs + off.vofs(db, 0) + ps * 16 * 2 * D));
                const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4_t *)(Vs + off.vofs(db, 1) + ps * 16 * 2 * D));
                const u32x2_t lw = __builtin_bit_cast(u32x2_t, lo);
                const u32x2_t hw = __builtin_bit_cast(u32x2_t, hi);
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, (u32x4_t){lw[0], lw[1], hw[0], hw[1]});
                o[db] = mfma32(a, pb, o[db]);
            }
        }
    }
};

// Wait until at most `ahead` tiles of copies (LPT loads each) are in flight:
// the oldest tile has landed.  gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14,
// expcnt 7 and lgkmcnt 15 (no wait on those).
template <int LPT, int MAXA>
__device__ __forceinline__ void wait_tiles_ahead(int ahead)
{
#define FA_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | 0x0F70)
    static_assert(MAXA * LPT <= 63, "vmcnt holds at most 63");
    if (MAXA >= 3 && ahead >= 3) __builtin_amdgcn_s_waitcnt(FA_VMCNT(3 * LPT));
    else if (MAXA >= 2 && ahead >= 2) __builtin_amdgcn_s_waitcnt(FA_VMCNT(2 * LPT));
    else if (MAXA >= 1 && ahead >= 1) __builtin_amdgcn_s_waitcnt(FA_VMCNT(LPT));
    else wait_vmem();
#undef FA_VMCNT
}

// One step of the split-key decode loop over an S-stage LDS ring: tile n sits
// in stage `st` (= n % S); tiles n + 1 .. n + S - 2 may still be in flight;
// the copies of tile n + S - 1 start into the stage tile n - 1 used.
template <int D, int BN, int S, class LD>
__device__ __forceinline__ void decode_step(
    int n, int n_tiles, int key_base, char *lds, int st, const LD &ld,
    int lane, int key_end, int wmin_lim, const OperandOffsets<D> &off,
    const bf16x8_t (&qf)[D / 16], f32x16_t (&o)[D / 32], float &m_ref, float &l_run,
    float &l_rnd, float c, int half, int lim_lane)
{
    constexpr int TB = LD::TILE_BYTES;
    constexpr int STAGE = 2 * TB;
    constexpr int LPT = 2 * LD::PER_WAVE;
    const int ahead = min(S - 2, n_tiles - 1 - n);
    wait_tiles_ahead<LPT, S - 2>(ahead);
    // one wave: orders its LDS reads of tile n - 1 before the copies below
    // overwrite that stage
    __syncthreads();
    if (n + S - 1 < n_tiles) {
        char *dst = lds + ((st + S - 1) % S) * STAGE;
        ld.issue(dst, dst + TB, key_base + (n + S - 1) * BN, 0, lane);
    }
    const char *stage = lds + st * STAGE;
    const int key0 = key_base + n * BN;
    // one (masked) copy of the step at D = 256: two inlined copies there
    // keep two register assignments of O alive and spill
    const bool need_mask = D >= 256 || (key0 + BN > key_end) || (key0 + BN - 1 > wmin_lim);
    if (need_mask)
        WaveTile<D, BN>::template step<true>(stage, stage + TB, off, qf, o, m_ref, l_run, l_rnd,
                                             c, half, key0, key_end, lim_lane);
    else
        WaveTile<D, BN>::template step<false>(stage, stage + TB, off, qf, o, m_ref, l_run, l_rnd,
                                              c, half, key0, key_end, lim_lane);
}

// Load this lane's Q fragment (B operand of S^T = K Q^T): head dims
// 16*st + 8*half .. +7 of one query row, for st = 0..D/16-1.  The loads go
// straight into the fragment registers, all issued before anything waits on
// them (callers issue their first K/V copies before this, so one memory round
// trip covers both).  Callers pass an in-range row: rows past the problem
// load the last real row, whose columns are never written.
template <int D>
__device__ __forceinline__ void load_q(bf16x8_t (&qf)[D / 16], const uint16_t *qrow, int half)
{
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
        qf[st] = __builtin_bit_cast(bf16x8_t, ld16(qrow + 16 * st + 8 * half));
}

// A negative scale is applied by negating Q exactly (sign bits), once the
// fragment has landed.  The empty asm reads every fragment register on every
// path: the compiler then knows the loads are complete before the key loop,
// instead of re-waiting on them (vmcnt, which would also drain the K/V copies
// in flight) at each S MFMA.
template <int D>
__device__ __forceinline__ void flip_q(bf16x8_t (&qf)[D / 16], uint32_t qflip)
{
    if (qflip) {
#pragma unroll
        for (int st = 0; st < D / 16; ++st)
            qf[st] = __builtin_bit_cast(bf16x8_t, __builtin_bit_cast(u32x4_t, qf[st]) ^ qflip);
    }
#pragma unroll
    for (int st = 0; st < D / 16; ++st) asm volatile("" ::"v"(qf[st]));
}

// Store a wave's 32 transposed rows (lane (col, half), register r of block db
// = element 32 db + 8 (r / 4) + 4 half + r % 4 of row col) times `mult` at
// out + obase, as bf16 (round to nearest even) or fp32.  All values first,
// each store's data in registers of its own, then the stores back to back:
// rewriting a store's data registers right behind it stalls the wave until
// the store has read them.
template <int D, bool OUT_F32>
__device__ __forceinline__ void store_rows(const f32x16_t (&o)[D / 32], float mult, int half,
                                           void *out, long obase)
{
    if (OUT_F32) {
        f32x4_t ov[D / 32][4];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
                ov[db][gq] = (f32x4_t){o[db][4 * gq] * mult, o[db][4 * gq + 1] * mult,
                                       o[db][4 * gq + 2] * mult, o[db][4 * gq + 3] * mult};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
                *reinterpret_cast<f32x4_t *>(static_cast<float *>(out) + obase + db * 32 + 8 * gq +
                                             4 * half) = ov[db][gq];
    } else {
        // bf16: a lane holds 4 consecutive elements per (db, gq) and its
        // partner in the other lane half the next 4.  One lane-half swap per
        // register pair gives the lower half 8 consecutive elements of gq
        // 2m and the upper half those of gq 2m + 1: half as many stores,
        // 16 bytes each.
        u32x4_t ov[D / 32][2];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int ga = 2 * m, gb = 2 * m + 1;
                const uint32_t a0 = pack_bf16(o[db][4 * ga] * mult, o[db][4 * ga + 1] * mult);
                const uint32_t a1 = pack_bf16(o[db][4 * ga + 2] * mult, o[db][4 * ga + 3] * mult);
                const uint32_t b0 = pack_bf16(o[db][4 * gb] * mult, o[db][4 * gb + 1] * mult);
                const uint32_t b1 = pack_bf16(o[db][4 * gb + 2] * mult, o[db][4 * gb + 3] * mult);
                // lower lanes: (own a, upper partner's a); upper lanes: (lower
                // partner's b, own b)
                const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
                ov[db][m] = (u32x4_t){s0[0], s1[0], s0[1], s1[1]};
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int m = 0; m < 2; ++m)
                *reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(out) + obase + db * 32 +
                                             16 * m + 8 * half) = ov[db][m];
    }
}

// Epilogue of one wave's 32 query columns: O = O / l_norm, and
// LSE = ln 2 * (c*m + log2 l) from the exact row sum l.  l_norm (whole row)
// is the sum of the rounded P that O accumulated; l_part is this lane
// half's share of the exact sum.
template <int D, bool OUT_F32>
__device__ __forceinline__ void finish_rows(const f32x16_t (&o)[D / 32], float m_ref,
                                            float l_part, float l_norm, float c, int half,
                                            void *out, long obase, float *lse_out, bool write)
{
    const float l = add_halves(l_part);
    const float inv = l_norm > 0.0f ? 1.0f / l_norm : 0.0f;
    if (!write) return;
    store_rows<D, OUT_F32>(o, inv, half, out, obase);
    if (lse_out && half == 0) {
        const float mc = (m_ref == kNegInf) ? 0.0f : m_ref * c;
        *lse_out = l > 0.0f ? (mc + __log2f(l)) * kLn2 : kNegInf;
    }
}

// ---------------------------------------------------------------------------
// Per-block pieces of the pipelined prefill (a block = 32 keys).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A operand that turns a 16x16x32 MFMA into per-query row sums of P.  Fed to
// that MFMA, the P registers of a 32x32x16 step (B operand) are read as: lane
// group h = lane / 16 holds column lane % 16 and k-group h, so lane 16h + c
// carries query c + 16 (h % 2) and one half of the step's 16 keys.  An A
// operand that is one where (lane group) % 2 == (row / 4) % 2 and zero
// elsewhere therefore makes accumulator rows 4h .. 4h+3 of column c the sum
// over all 16 keys of query c + 16 (h % 2).  In the 16x16 accumulator layout
// (lane 16h + c holds rows 4h .. 4h+3 of column c) that is the lane's own
// query, the same one its 32x32 registers belong to.
__device__ __forceinline__ bf16x8_t rowsum_selector(int lane)
{
    const bool on = ((lane >> 4) & 1) == ((lane >> 2) & 1);
    const uint32_t w = on ? 0x3f803f80u : 0u;
    return __builtin_bit_cast(bf16x8_t, (u32x4_t){w, w, w, w});
}

template <int D>
struct BlockOps {
    static constexpr int QS = D / 16;
    static constexpr int DB = D / 32;
    // At D = 256 a wave has its SIMD to itself (one workgroup per CU), so a
    // priority has nothing to order; left out there, the compiler may
    // schedule the softmax's VALU work between the MFMAs (+1.4 % measured).
    static constexpr bool kPrio = D < 256;

    // S^T of one 32-key block whose K rows start at Kblk (LDS).
    __device__ __forceinline__ static f32x16_t qk(const char *Kblk, const OperandOffsets<D> &off,
                                                  const bf16x8_t (&qf)[QS])
    {
        f32x16_t s = f32x16_t{};
        set_prio<1, kPrio>();
#pragma unroll
        for (int st = 0; st < QS; ++st) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(Kblk + off.kofs(st));
            s = mfma32(a, qf[st], s);
        }
        set_prio<0, kPrio>();
        return s;
    }

    // keys >= key_end, or beyond this lane's causal limit, score -inf.
    // Register r holds key key0 + 4*half + 8*(r/4) + r%4; comparing the
    // constant part against one per-lane bound keeps the 16 offsets as
    // instruction immediates (no registers to hold, or spill, them in).
    // Selects, not conditional assignments: written as `if (...) s[r] = -inf`
    // the compiler turned the mask into a branch on the lane's limit (skip
    // when nothing is masked), and the register allocator then placed copies
    // of loop-carried values (the exact row sums) inside that branch, where
    // the lanes that skipped it never received them.
    __device__ __forceinline__ static void mask(f32x16_t &s, int key0, int half, int key_end,
                                                int lim)
    {
        const int base = key0 + 4 * half;
        const int last = min(lim, key_end - 1) - base;   // largest allowed offset
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = (8 * (r >> 2) + (r & 3) > last) ? kNegInf : s[r];
    }

    // max over the block's keys of this lane's query (both lane halves)
    __device__ __forceinline__ static float rowmax(const f32x16_t &s)
    {
        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        return max_halves(mx);
    }

    // Lazy reference max: move it (and rescale O and l) only for rows whose
    // max grew past the threshold; the first allowed key always does.
    __device__ __forceinline__ static void rebase(float mx, float &m_ref, float &l_run,
                                                  f32x4_t &l_acc, f32x16_t (&o)[DB], float c)
    {
        const bool grow = (mx - m_ref) * c > kRescaleThreshold;
        if (__any(grow)) {
            const float m_new = grow ? mx : m_ref;
            const float alpha = (m_ref == kNegInf) ? 0.0f : fast_exp2((m_ref - m_new) * c);
            l_run *= alpha;
            l_acc[0] *= alpha;   // only element 0 of the row-sum accumulator is read
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
            m_ref = m_new;
        }
    }

    // P = exp2(c*s - mc), rounded to bf16, as the B operands of the block's two
    // 16-key PV steps (p0: registers 0..7, p1: 8..15).  l_run adds the exact
    // fp32 values (it feeds the LSE); the sum of the rounded values, which
    // normalises O, is taken on the MFMA unit in pv().
    template <bool MASK>
    __device__ __forceinline__ static void probs(const f32x16_t &s, float c, float mc,
                                                 bf16x8_t &p0, bf16x8_t &p1, float &l_run)
    {
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            e[r] = fast_exp2(fmaf(s[r], c, -mc));
            if (MASK) e[r] = (s[r] == kNegInf) ? 0.0f : e[r];
        }
        u32x4_t w0, w1;
        float la = 0.0f, lb = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            w0[q] = pack_bf16(e[2 * q], e[2 * q + 1]);
            w1[q] = pack_bf16(e[8 + 2 * q], e[8 + 2 * q + 1]);
            la += e[2 * q] + e[2 * q + 1];
            lb += e[8 + 2 * q] + e[8 + 2 * q + 1];
        }
        l_run += la + lb;
        p0 = __builtin_bit_cast(bf16x8_t, w0);
        p1 = __builtin_bit_cast(bf16x8_t, w1);
    }

    // O^T += V^T P^T over the block whose V rows start at Vblk (LDS).  The
    // same P also meets the row-sum selector: l_acc then holds the running
    // sum of the rounded P of this lane's query -- the values P V multiplies,
    // so O / sum is normalised consistently (with the lazy reference P
    // reaches 2^8 and is not exact in bf16; a dominant key's rounding then
    // divides out).
    __device__ __forceinline__ static void pv(const char *Vblk, const OperandOffsets<D> &off,
                                              bf16x8_t sel, bf16x8_t p0, bf16x8_t p1,
                                              f32x16_t (&o)[DB], f32x4_t &l_acc)
    {
        set_prio<1, kPrio>();
        l_acc = mfma16(sel, p0, l_acc);
        l_acc = mfma16(sel, p1, l_acc);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4_t *)(Vblk + off.vofs(db, 0) + t2 * 16 * 2 * D));
                const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4_t *)(Vblk + off.vofs(db, 1) + t2 * 16 * 2 * D));
                const u32x2_t lw = __builtin_bit_cast(u32x2_t, lo);
                const u32x2_t hw = __builtin_bit_cast(u32x2_t, hi);
                const bf16x8_t a =
                    __builtin_bit_cast(bf16x8_t, (u32x4_t){lw[0], lw[1], hw[0], hw[1]});
                o[db] = mfma32(a, t2 ? p1 : p0, o[db]);
            }
        }
        set_prio<0, kPrio>();
    }
};

// State of one wave's query rows while the workgroup walks the key tiles.
template <int D>
struct RowState {
    bf16x8_t qf[D / 16];
    f32x16_t o[D / 32];
    f32x16_t s_cur;      // S^T of the block to be finished next
    float mx_cur;        // its row max
    float m_ref, l_run;  // lazy reference max and exact row sum (this lane half)
    f32x4_t l_acc;       // element 0: row sum of the rounded P (whole row)
    bf16x8_t sel;        // row-sum selector operand
    int NBw;             // blocks this wave has work on (a prefix of the tile walk)
    int wmin_lim;        // smallest causal limit of the wave's rows
    int lim_lane;        // this lane's causal limit
    int key_end;
    int half;
    float c;

    __device__ __forceinline__ bool needs_mask(int j) const
    {
        return (j * 32 + 32 > key_end) || (j * 32 + 31 > wmin_lim);
    }
};

// The blocks of tile t (held in LDS stage `stage`).  Pipeline: while block j
// is finished (softmax, P V) the S^T of block j + 1 is already issued, so the
// MFMA and VALU work of neighbouring blocks overlap.  Block j + 1 may be the
// first block of tile t + 1 (stage `next`): the barrier that makes tile t + 1
// ready is taken first, and tile t + 2's copies then start into `after`, the
// stage tile t - 1 used, which every wave has finished by that barrier.
template <int D, int BN, int NW>
__device__ __forceinline__ void prefill_tile(int t, int n_tiles, char *stage, char *next,
                                             char *after, const TileLoader<D, BN, NW> &ld,
                                             int wave, int lane, const OperandOffsets<D> &off,
                                             RowState<D> &rs)
{
    constexpr int KB = BN / 32;
    constexpr int TB = TileLoader<D, BN, NW>::TILE_BYTES;
    using BO = BlockOps<D>;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int j = t * KB + kb;
        const bool live = j < rs.NBw;
        const bool live_next = j + 1 < rs.NBw;
        float mc = 0.0f;
        if (live) {
            BO::rebase(rs.mx_cur, rs.m_ref, rs.l_run, rs.l_acc, rs.o, rs.c);
            mc = (rs.m_ref == kNegInf) ? 0.0f : rs.m_ref * rs.c;
        }
        const char *Knext = stage + (kb + 1) * 32 * 2 * D;
        if (kb == KB - 1) {
            Knext = next;
            if (t + 1 < n_tiles) {
                wait_vmem();       // this wave's copies of tile t + 1 are in LDS
                __syncthreads();   // ... and every wave's; tile t - 1 is released
                if (t + 2 < n_tiles) ld.issue(after, after + TB, (t + 2) * BN, wave, lane);
            }
        }
        f32x16_t s_next = f32x16_t{};
        if (live_next) s_next = BO::qk(Knext, off, rs.qf);
        if (live) {
            bf16x8_t p0, p1;
            if (rs.needs_mask(j))
                BO::template probs<true>(rs.s_cur, rs.c, mc, p0, p1, rs.l_run);
            else
                BO::template probs<false>(rs.s_cur, rs.c, mc, p0, p1, rs.l_run);
            BO::pv(stage + TB + kb * 32 * 2 * D, off, rs.sel, p0, p1, rs.o, rs.l_acc);
        }
        if (live_next) {
            if (rs.needs_mask(j + 1))
                BO::mask(s_next, (j + 1) * 32, rs.half, rs.key_end, rs.lim_lane);
            rs.mx_cur = BO::rowmax(s_next);
        }
        rs.s_cur = s_next;
    }
}

// ---------------------------------------------------------------------------
// Prefill: one workgroup = NW waves = 32*NW query rows of one (b, hq); K/V
// tiles of BN keys stream through a three-stage LDS ring filled by
// HBM -> LDS copies, one barrier per tile.
// ---------------------------------------------------------------------------
template <int D, int BN, int NW, bool OUT_F32>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
fa_prefill_kernel(const Params p)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    constexpr int BM = 32 * NW;
    constexpr int KB = BN / 32;
    using TL = TileLoader<D, BN, NW>;
    using BO = BlockOps<D>;
    constexpr int TB = TL::TILE_BYTES;
    constexpr int STAGE = 2 * TB;   // K tile then V tile

    __shared__ __attribute__((aligned(1024))) char lds[kPrefillStages * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the wave index is uniform across the wave: say so, so that everything
    // derived from it (tile-copy descriptors, row ranges) stays scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;

    OperandOffsets<D> off;
    off.init(lane);

    const int BH = p.B * p.Hq;
    const int ND = p.domains;
    const int x = blockIdx.x % ND;           // scheduling domain (XCD)
    const int jw = blockIdx.x / ND;          // workgroup index inside the domain
    const int Gx = gridDim.x / ND;
    const int BHx = BH / ND;                 // (b, hq) pairs of this domain
    const int Nx = BHx * p.n_mblocks;        // items of this domain

    for (int it = 0; it * Gx < Nx; ++it) {
        const int li = it * Gx + ((it & 1) ? (Gx - 1 - jw) : jw);
        if (li >= Nx) continue;
        // rank-major: all heads' longest blocks first; head-major: all
        // blocks of one head before the next, so that more workgroups of an
        // XCD stream the same K/V at once.  Either way the snake over it
        // balances the causal lengths.
        const int rank = p.head_major ? li % p.n_mblocks : li / BHx;
        const int bh = (p.head_major ? li / p.n_mblocks : li % BHx) * ND + x;
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

        RowState<D> rs;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) rs.o[db] = f32x16_t{};
        rs.m_ref = kNegInf;
        rs.l_run = 0.0f;
        rs.l_acc = f32x4_t{};
        rs.sel = rowsum_selector(lane);
        rs.s_cur = f32x16_t{};
        rs.mx_cur = kNegInf;
        rs.half = half;
        rs.c = p.c;
        rs.key_end = p.Sk;
        rs.lim_lane = p.causal ? qi + p.off : 0x7fffffff;
        rs.wmin_lim = p.causal ? wrow0 + p.off : 0x7fffffff;
        const int NB = n_tiles * KB;
        if (wrow0 >= p.Sq)
            rs.NBw = 0;
        else if (p.causal) {
            const int wmax_lim = wlast + p.off;          // largest limit of the wave
            rs.NBw = wmax_lim < 0 ? 0 : min(NB, wmax_lim / 32 + 1);
        } else
            rs.NBw = NB;

        TL ld;
        ld.setup(p.k + ((long)b * p.Sk * p.Hkv + g) * D, p.v + ((long)b * p.Sk * p.Hkv + g) * D,
                 p.Hkv * D * 2, p.Sk);

        // the first two tiles' copies, then Q: one memory round trip for all
        if (n_tiles > 0) ld.issue(lds, lds + TB, 0, wave, lane);
        if (n_tiles > 1) ld.issue(lds + STAGE, lds + STAGE + TB, BN, wave, lane);
        load_q<D>(rs.qf, p.q + (((long)b * p.Sq + min(qi, p.Sq - 1)) * p.Hq + hq) * D, half);
        wait_vmem();
        flip_q<D>(rs.qf, p.qflip);
        if (n_tiles > 0) {
            __syncthreads();
            if (rs.NBw > 0) {
                rs.s_cur = BO::qk(lds, off, rs.qf);
                if (rs.needs_mask(0)) BO::mask(rs.s_cur, 0, half, rs.key_end, rs.lim_lane);
                rs.mx_cur = BO::rowmax(rs.s_cur);
            }
        }
        // tile t lives in stage t % 3; three tiles per trip keep every LDS
        // offset a compile-time constant
        for (int t = 0; t < n_tiles; t += 3) {
            prefill_tile<D, BN, NW>(t, n_tiles, lds, lds + STAGE, lds + 2 * STAGE, ld, wave, lane,
                                    off, rs);
            if (t + 1 < n_tiles)
                prefill_tile<D, BN, NW>(t + 1, n_tiles, lds + STAGE, lds + 2 * STAGE, lds, ld,
                                        wave, lane, off, rs);
            if (t + 2 < n_tiles)
                prefill_tile<D, BN, NW>(t + 2, n_tiles, lds + 2 * STAGE, lds, lds + STAGE, ld,
                                        wave, lane, off, rs);
        }
        __syncthreads();   // every wave is done with the LDS ring before the next item

        finish_rows<D, OUT_F32>(rs.o, rs.m_ref, rs.l_run, rs.l_acc[0], p.c, half, p.o,
                                (((long)b * p.Sq + qi) * p.Hq + hq) * D,
                                p.lse ? p.lse + ((long)b * p.Hq + hq) * p.Sq + qi : nullptr,
                                qi < p.Sq);
    }
#endif
}

// ---------------------------------------------------------------------------
// FP8 E4M3 prefill: Q, K, V as OCP E4M3 codes with per-tensor descales.
// S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x64_f8f6f4 (64 keys
// or head dims per instruction, twice the bf16 rate), P is rounded to E4M3.
// Lane layout of that MFMA: A lane (m = lane % 32, h = lane / 32) holds
// A[m][32h .. 32h + 31], B lane (n, h) holds B[32h .. 32h + 31][n]; the
// output is laid out as for the bf16 32x32 MFMAs.
//
// One block is 64 keys, two 32-key S^T accumulators: lane (col, h) holds,
// in accumulator kb register r, key kb*32 + 8*(r/4) + 4h + r%4 =: key(h, i)
// with i = 16 kb + r.  Packed to E4M3 in that order (byte i), they are
// directly the B operand P^T of the PV product if the A operand V^T holds
// V[key(h, i)][dim] at byte i.  ds_read_b64_tr_b8 delivers exactly that:
// in each group of 16 lanes, lane j receives byte j % 8 of the 8-byte words
// the group's lanes 2t + j / 8 point at (t = 0..7, output byte t), so a
// source lane s points at the 8 dims it shares with its destinations in key
// row key(h, 8 t4 + s / 2), for the read t4 = 0..3 of the 32 bytes.
// Tiles are rows of D bytes: the bf16 geometry of head dim D/2 (loader,
// swizzle), so both reads stay conflict-free as there.
// ---------------------------------------------------------------------------
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

__device__ __forceinline__ f32x16_t mfma32_f8(i32x8_t a, i32x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int D>
struct Fp8Offsets {
    static constexpr int RB = D;          // bytes per tile row
    static constexpr int KS = D / 64;     // k-steps of S^T
    static constexpr int DB = D / 32;     // 32-dim blocks of O^T
    int k[KS][2];                         // the two 16-byte chunks of a k-step (+ kb*32 rows)
    int vb[4];                            // read t4: this lane's source row and byte offset
    int vs[4];                            //   and its row's swizzle / 2

    // Address of this lane's 8 source bytes for read t4 of dim block db: the
    // chunk (2 db + grp % 2) ^ swz(key) is split into its low bit (kept in
    // vb) and 2 (db ^ swz/2), so that four registers serve every db.
    __device__ __forceinline__ int vofs(int db, int t4) const { return vb[t4] + 32 * (db ^ vs[t4]); }

    __device__ __forceinline__ void init(int lane)
    {
        const int col = lane & 31, half = lane >> 5;
#pragma unroll
        for (int st = 0; st < KS; ++st)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const int chunk = 4 * st + 2 * half + c2;
                k[st][c2] = col * RB + ((chunk ^ swz_fp8(col)) * 16);
            }
        const int sl = lane & 15, grp = lane >> 4;
        static_assert(D == 128, "vofs assumes 8 chunks per row (4 dim blocks)");
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const int i = 8 * t4 + (sl >> 1);
            const int r = i & 15;
            const int key = (i >> 4) * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            const int sw = swz_fp8(key);
            vb[t4] = key * RB + 16 * ((grp ^ sw) & 1) + 8 * (sl & 1);
            vs[t4] = sw >> 1;
        }
    }
};

template <int D>
struct Fp8Ops {
    static constexpr int KS = D / 64;
    static constexpr int DB = D / 32;
    static constexpr int RB = D;

    // S^T of the 64 keys whose K rows start at Kblk (LDS)
    __device__ __forceinline__ static void qk(const char *Kblk, const Fp8Offsets<D> &off,
                                              const i32x8_t (&qf)[KS], f32x16_t (&s)[2])
    {
        set_prio<1>();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16_t{};
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                const u32x4_t lo =
                    *reinterpret_cast<const u32x4_t *>(Kblk + kb * 32 * RB + off.k[st][0]);
                const u32x4_t hi =
                    *reinterpret_cast<const u32x4_t *>(Kblk + kb * 32 * RB + off.k[st][1]);
                const i32x8_t a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                s[kb] = mfma32_f8(a, qf[st], s[kb]);
            }
        }
        set_prio<0>();
    }

    __device__ __forceinline__ static void mask(f32x16_t (&s)[2], int key0, int half,
                                                int key_end, int lim)
    {
        BlockOps<64>::mask(s[0], key0, half, key_end, lim);
        BlockOps<64>::mask(s[1], key0 + 32, half, key_end, lim);
    }

    __device__ __forceinline__ static float rowmax(const f32x16_t (&s)[2])
    {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        return max_halves(mx);
    }

    // Lazy reference max (threshold 2^8: P stays below 2^8, inside E4M3's
    // range of 448); the first allowed key always moves it.
    __device__ __forceinline__ static void rebase(float mx, float &m_ref, float &l_run,
                                                  f32x16_t &l_acc, f32x16_t (&o)[DB], float c)
    {
        const bool grow = (mx - m_ref) * c > kRescaleThreshold;
        if (__any(grow)) {
            const float m_new = grow ? mx : m_ref;
            const float alpha = (m_ref == kNegInf) ? 0.0f : fast_exp2((m_ref - m_new) * c);
            l_run *= alpha;
            l_acc[0] *= alpha;   // only element 0 of the row-sum accumulator is read
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
            m_ref = m_new;
        }
    }

    // P = exp2(c*s - mc) rounded to E4M3 (round to nearest even), byte
    // 16 kb + r of the B operand; l_run adds the exact fp32 values (LSE).
    template <bool MASK>
    __device__ __forceinline__ static i32x8_t probs(const f32x16_t (&s)[2], float c, float mc,
                                                    float &l_run)
    {
        float e[32];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = fast_exp2(fmaf(s[kb][r], c, -mc));
                if (MASK) x = (s[kb][r] == kNegInf) ? 0.0f : x;
                e[16 * kb + r] = x;
            }
        i32x8_t pw;
        float la = 0.0f, lb = 0.0f;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(e[4 * w], e[4 * w + 1], 0, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(e[4 * w + 2], e[4 * w + 3], word, true);
            pw[w] = word;
            la += e[4 * w] + e[4 * w + 1];
            lb += e[4 * w + 2] + e[4 * w + 3];
        }
        l_run += la + lb;
        return pw;
    }

    // O^T += V^T P^T over the 64 keys whose V rows start at Vblk; l_acc
    // (element 0) adds the column sums of the rounded P: the row sum O is
    // normalised by, from the same values P V multiplies.
    __device__ __forceinline__ static void pv(const char *Vblk, const Fp8Offsets<D> &off,
                                              i32x8_t pw, f32x16_t (&o)[DB], f32x16_t &l_acc)
    {
        constexpr int kOnes = 0x38383838;   // E4M3 1.0 in every byte
        const i32x8_t ones = {kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes};
        set_prio<1>();
        l_acc = mfma32_f8(ones, pw, l_acc);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            i32x8_t a;
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
                const i32x2_t w =
                    __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t *)(Vblk + off.vofs(db, t4)));
                a[2 * t4] = w[0];
                a[2 * t4 + 1] = w[1];
            }
            o[db] = mfma32_f8(a, pw, o[db]);
        }
        set_prio<0>();
    }
};

template <int D>
struct Fp8RowState {
    i32x8_t qf[D / 64];
    f32x16_t o[D / 32];
    f32x16_t s_cur[2];   // S^T of the block to be finished next
    float mx_cur;
    float m_ref, l_run;
    f32x16_t l_acc;      // element 0: row sum of the rounded P (whole row)
    int NBw, wmin_lim, lim_lane, key_end, half;
    float c;

    __device__ __forceinline__ bool needs_mask(int j) const
    {
        return (j * 64 + 64 > key_end) || (j * 64 + 63 > wmin_lim);
    }
};

// Tile t (64 keys, one block) held in LDS stage `stage`; the S^T of block
// t + 1 is issued before block t is finished, as in prefill_tile.
template <int D, int NW>
__device__ __forceinline__ void prefill_tile_fp8(int t, int n_tiles, char *stage, char *next,
                                                 char *after,
                                                 const TileLoader<D / 2, 64, NW, false, true> &ld,
                                                 int wave,
                                                 int lane, const Fp8Offsets<D> &off,
                                                 Fp8RowState<D> &rs)
{
    constexpr int TB = TileLoader<D / 2, 64, NW, false, true>::TILE_BYTES;
    using FO = Fp8Ops<D>;
    const bool live = t < rs.NBw;
    const bool live_next = t + 1 < rs.NBw;
    float mc = 0.0f;
    if (live) {
        FO::rebase(rs.mx_cur, rs.m_ref, rs.l_run, rs.l_acc, rs.o, rs.c);
        mc = (rs.m_ref == kNegInf) ? 0.0f : rs.m_ref * rs.c;
    }
    if (t + 1 < n_tiles) {
        wait_vmem();       // this wave's copies of tile t + 1 are in LDS
        __syncthreads();   // ... and every wave's; tile t - 1 is released
        if (t + 2 < n_tiles) ld.issue(after, after + TB, (t + 2) * 64, wave, lane);
    }
    f32x16_t s_next[2] = {f32x16_t{}, f32x16_t{}};
    if (live_next) FO::qk(next, off, rs.qf, s_next);
    if (live) {
        const i32x8_t pw = rs.needs_mask(t)
                               ? FO::template probs<true>(rs.s_cur, rs.c, mc, rs.l_run)
                               : FO::template probs<false>(rs.s_cur, rs.c, mc, rs.l_run);
        FO::pv(stage + TB, off, pw, rs.o, rs.l_acc);
    }
    if (live_next) {
        if (rs.needs_mask(t + 1)) FO::mask(s_next, (t + 1) * 64, rs.half, rs.key_end, rs.lim_lane);
        rs.mx_cur = FO::rowmax(s_next);
    }
    rs.s_cur[0] = s_next[0];
    rs.s_cur[1] = s_next[1];
}

template <int D, int NW, bool OUT_F32>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW == 8 ? 2 : 1)))
fa_prefill_fp8_kernel(const Params p, const float v_descale)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    constexpr int BN = 64;
    constexpr int BM = 32 * NW;
    using TL = TileLoader<D / 2, BN, NW, false, true>;
    using FO = Fp8Ops<D>;
    constexpr int TB = TL::TILE_BYTES;
    constexpr int STAGE = 2 * TB;

    __shared__ __attribute__((aligned(1024))) char lds[kPrefillStages * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;

    Fp8Offsets<D> off;
    off.init(lane);

    const uint8_t *q8 = reinterpret_cast<const uint8_t *>(p.q);
    const uint8_t *k8 = reinterpret_cast<const uint8_t *>(p.k);
    const uint8_t *v8 = reinterpret_cast<const uint8_t *>(p.v);

    const int BH = p.B * p.Hq;
    const int ND = p.domains;
    const int x = blockIdx.x % ND;
    const int jw = blockIdx.x / ND;
    const int Gx = gridDim.x / ND;
    const int BHx = BH / ND;
    const int Nx = BHx * p.n_mblocks;

    for (int it = 0; it * Gx < Nx; ++it) {
        const int li = it * Gx + ((it & 1) ? (Gx - 1 - jw) : jw);
        if (li >= Nx) continue;
        const int rank = p.head_major ? li % p.n_mblocks : li / BHx;
        const int bh = (p.head_major ? li / p.n_mblocks : li % BHx) * ND + x;
        const int mb = p.causal ? (p.n_mblocks - 1 - rank) : rank;
        const int b = bh / p.Hq;
        const int hq = bh % p.Hq;
        const int g = hq / p.group;

        const int row0 = mb * BM;
        const int wrow0 = row0 + wave * 32;
        const int qi = wrow0 + col;
        const int last_row = min(row0 + BM, p.Sq) - 1;
        const int wlast = min(wrow0 + 31, p.Sq - 1);

        int n_tiles = (p.Sk + BN - 1) / BN;
        if (p.causal) {
            const int hi = last_row + p.off;
            n_tiles = hi < 0 ? 0 : min(n_tiles, hi / BN + 1);
        }

        Fp8RowState<D> rs;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) rs.o[db] = f32x16_t{};
        rs.m_ref = kNegInf;
        rs.l_run = 0.0f;
        rs.l_acc = f32x16_t{};
        rs.s_cur[0] = f32x16_t{};
        rs.s_cur[1] = f32x16_t{};
        rs.mx_cur = kNegInf;
        rs.half = half;
        rs.c = p.c;
        rs.key_end = p.Sk;
        rs.lim_lane = p.causal ? qi + p.off : 0x7fffffff;
        rs.wmin_lim = p.causal ? wrow0 + p.off : 0x7fffffff;
        if (wrow0 >= p.Sq)
            rs.NBw = 0;
        else if (p.causal) {
            const int wmax_lim = wlast + p.off;
            rs.NBw = wmax_lim < 0 ? 0 : min(n_tiles, wmax_lim / BN + 1);
        } else
            rs.NBw = n_tiles;

        TL ld;
        ld.setup(reinterpret_cast<const uint16_t *>(k8 + ((long)b * p.Sk * p.Hkv + g) * D),
                 reinterpret_cast<const uint16_t *>(v8 + ((long)b * p.Sk * p.Hkv + g) * D),
                 p.Hkv * D, p.Sk);

        // the first keys of tiles 0 and 1 behind opaque values: their copy
        // offsets are formed here, not precomputed for the kernel and spilled
        // (each reload waits, vmcnt(0), for every copy and store before it)
        int k0 = 0, k1 = BN;
        asm volatile("" : "+s"(k0), "+s"(k1));
        if (n_tiles > 0) ld.issue(lds, lds + TB, k0, wave, lane);
        if (n_tiles > 1) ld.issue(lds + STAGE, lds + STAGE + TB, k1, wave, lane);
        {
            // this lane's Q bytes: k-step st, dims 64 st + 32 half .. + 31
            const uint8_t *qrow = q8 + (((long)b * p.Sq + min(qi, p.Sq - 1)) * p.Hq + hq) * D;
#pragma unroll
            for (int st = 0; st < D / 64; ++st) {
                const u32x4_t lo = ld16(reinterpret_cast<const uint16_t *>(qrow + 64 * st + 32 * half));
                const u32x4_t hi =
                    ld16(reinterpret_cast<const uint16_t *>(qrow + 64 * st + 32 * half + 16));
                rs.qf[st] = (i32x8_t){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
        }
        wait_vmem();
        // a negative scale negates Q exactly (E4M3 sign bits)
#pragma unroll
        for (int st = 0; st < D / 64; ++st) {
            if (p.qflip) rs.qf[st] ^= (int)0x80808080u;
            asm volatile("" ::"v"(rs.qf[st]));
        }
        if (n_tiles > 0) {
            __syncthreads();
            if (rs.NBw > 0) {
                FO::qk(lds, off, rs.qf, rs.s_cur);
                if (rs.needs_mask(0)) FO::mask(rs.s_cur, 0, half, rs.key_end, rs.lim_lane);
                rs.mx_cur = FO::rowmax(rs.s_cur);
            }
        }
        for (int t = 0; t < n_tiles; t += 3) {
            prefill_tile_fp8<D, NW>(t, n_tiles, lds, lds + STAGE, lds + 2 * STAGE, ld, wave, lane,
                                    off, rs);
            if (t + 1 < n_tiles)
                prefill_tile_fp8<D, NW>(t + 1, n_tiles, lds + STAGE, lds + 2 * STAGE, lds, ld,
                                        wave, lane, off, rs);
            if (t + 2 < n_tiles)
                prefill_tile_fp8<D, NW>(t + 2, n_tiles, lds + 2 * STAGE, lds, lds + STAGE, ld,
                                        wave, lane, off, rs);
        }
        __syncthreads();   // every wave is done with the LDS ring before the next item

        // O = v_descale * O / l: the descale folds into the normaliser
        finish_rows<D, OUT_F32>(rs.o, rs.m_ref, rs.l_run, rs.l_acc[0] / v_descale, p.c, half,
                                p.o, (((long)b * p.Sq + qi) * p.Hq + hq) * D,
                                p.lse ? p.lse + ((long)b * p.Hq + hq) * p.Sq + qi : nullptr,
                                qi < p.Sq);
    }
#endif
}

// ---------------------------------------------------------------------------
// Backward: dQ, dK, dV from Q, K, V, O, dO and the forward's LSE.
//   delta_i = sum_d dO_id O_id, kept negated                   (fa_bwd_delta_kernel)
//   P = exp(scale Q K^T - LSE), dP = dO V^T, dS = P (dP - delta)
//   dV = P^T dO, dK = scale dS^T Q                              (fa_bwd_dkdv_kernel)
//   dQ = scale dS K                                             (fa_bwd_dq_kernel)
// Two main kernels, each recomputing S and dP, so that every output element
// is owned by one wave (no atomics: results are deterministic).  Both use the
// forward's operand forms: one side of a product from registers (a row
// fragment), the other read from an LDS tile, and the transposed operand of
// the accumulating product read with the transposing LDS load in the key (or
// query) grouping of the accumulator registers, so that those registers,
// rounded to bf16, are its B operand directly.
// ---------------------------------------------------------------------------
struct BwdParams {
    const uint16_t *q, *k, *v, *o, *dout;
    const float *lse;
    float *ndelta;           // [B][Hq][Sq]: -rowsum(dO O)
    float *lse2;             // [B][Hq][Sq]: LSE * log2(e), +inf for rows without keys
    uint16_t *dq, *dk, *dv;
    int B, Hq, Hkv, Sq, Sk, group, causal, off;
    float c;          // |scale| * log2(e)
    float scale;      // signed, for dQ and dK
    uint32_t flip;    // 0x80008000 when scale < 0 (applied to the register fragment of S)
    int n_blocks;     // dkdv: key blocks per KV head; dq: query blocks per head
};

// ndelta[b][h][i] = -sum_d dO[b][i][h][d] * O[b][i][h][d] and lse2 = LSE log2 e,
// one row per thread.
template <int D>
__global__ void __launch_bounds__(256) fa_bwd_delta_kernel(const BwdParams p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    const long row = (long)blockIdx.x * 256 + threadIdx.x;   // (b, i, h), h fastest
    if (row >= (long)p.B * p.Sq * p.Hq) return;
    const uint16_t *orow = p.o + row * D;
    const uint16_t *drow = p.dout + row * D;
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < D; c += 8) {
        const u32x4_t a = ld16(orow + c), g = ld16(drow + c);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc = fmaf(__uint_as_float(a[w] << 16), __uint_as_float(g[w] << 16), acc);
            acc = fmaf(__uint_as_float(a[w] & 0xffff0000u), __uint_as_float(g[w] & 0xffff0000u),
                       acc);
        }
    }
    const int h = (int)(row % p.Hq);
    const long bi = row / p.Hq;
    const int i = (int)(bi % p.Sq);
    const int b = (int)(bi / p.Sq);
    const long vi = ((long)b * p.Hq + h) * p.Sq + i;
    p.ndelta[vi] = -acc;
    // exp(scale s - LSE) = exp2(c s - LSE log2 e); a row without keys has
    // LSE = -inf and must give P = 0
    const float l = p.lse[vi];
    p.lse2[vi] = l == kNegInf ? __builtin_inff() : l * 1.4426950408889634f;
#endif
}

// One HBM -> LDS copy of 4 bytes per lane for two vectors (same offsets, two
// descriptors, two LDS destinations): 64 floats each.
__device__ __forceinline__ void lds_dma4_pair(char *lds_a, char *lds_b, int voff, u32x4_t da,
                                              u32x4_t db)
{
    const uint32_t m0a = (uint32_t)reinterpret_cast<uintptr_t>((lds_void_t *)lds_a);
    const uint32_t m0b = (uint32_t)reinterpret_cast<uintptr_t>((lds_void_t *)lds_b);
    uint32_t saved;
    lds_check_before_copy<4>(lds_a);
    lds_check_before_copy<4>(lds_b);
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %3, %4, 0 offen lds\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %3, %5, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0a), "s"(m0b), "v"(voff), "s"(da), "s"(db)
        : "memory");
    lds_check_after_copy();
}

__device__ __forceinline__ u32x4_t raw_desc(const void *base, uint32_t nbytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return (u32x4_t){(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, nbytes, (uint32_t)kBufferFlags};
}

// The accumulating product of both kernels: acc^T += X^T Y^T over a 32-row
// block of an LDS tile (X rows at Xblk), Y^T the bf16 operand halves y0
// (registers 0..7 of the 32x32 accumulator) and y1 (8..15).
template <int D>
__device__ __forceinline__ void bwd_accumulate(const char *Xblk, const OperandOffsets<D> &off,
                                               bf16x8_t y0, bf16x8_t y1, f32x16_t (&acc)[D / 32])
{
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t *)(Xblk + off.vofs(db, 0) + t2 * 16 * 2 * D));
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t *)(Xblk + off.vofs(db, 1) + t2 * 16 * 2 * D));
            const u32x2_t lw = __builtin_bit_cast(u32x2_t, lo);
            const u32x2_t hw = __builtin_bit_cast(u32x2_t, hi);
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, (u32x4_t){lw[0], lw[1], hw[0], hw[1]});
            acc[db] = mfma32(a, t2 ? y1 : y0, acc[db]);
        }
    }
}

__device__ __forceinline__ void pack_halves(const float (&x)[16], bf16x8_t &y0, bf16x8_t &y1)
{
    u32x4_t w0, w1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        w0[q] = pack_bf16(x[2 * q], x[2 * q + 1]);
        w1[q] = pack_bf16(x[8 + 2 * q], x[8 + 2 * q + 1]);
    }
    y0 = __builtin_bit_cast(bf16x8_t, w0);
    y1 = __builtin_bit_cast(bf16x8_t, w1);
}

// dQ: one workgroup = NW waves x 32 query rows of one (b, hq); K/V tiles of
// 64 keys through the forward's three-stage ring.  Per 32-key block:
// S^T = K Q^T and dP^T = V dO^T (lane = query column: LSE and delta are
// lane-local), dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T.
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW == 8 ? 2 : 1)))
fa_bwd_dq_kernel(const BwdParams p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int BN = 64;
    constexpr int BM = 32 * NW;
    using TL = TileLoader<D, BN, NW>;
    using BO = BlockOps<D>;
    constexpr int TB = TL::TILE_BYTES;
    constexpr int STAGE = 2 * TB;
    __shared__ __attribute__((aligned(1024))) char lds[kPrefillStages * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;
    OperandOffsets<D> off;
    off.init(lane);

    // (b, hq) pairs in 8 residue classes, one per XCD (workgroup index mod 8),
    // when both counts allow: all blocks of a head then share one L2
    const int BH = p.B * p.Hq;
    const int ND = (BH % 8 == 0 && gridDim.x % 8 == 0) ? 8 : 1;
    const int x = blockIdx.x % ND;
    const int jw = blockIdx.x / ND;
    const int Gx = gridDim.x / ND;
    const int N = (BH / ND) * p.n_blocks;
    for (int it = 0; it * Gx < N; ++it) {
        const int li = it * Gx + ((it & 1) ? (Gx - 1 - jw) : jw);
        if (li >= N) continue;
        // head by head, each head's longest (causal: last) query blocks first
        const int bh = (li / p.n_blocks) * ND + x;
        const int rank = li % p.n_blocks;
        const int mb = p.causal ? (p.n_blocks - 1 - rank) : rank;
        const int b = bh / p.Hq;
        const int hq = bh % p.Hq;
        const int g = hq / p.group;
        const int row0 = mb * BM;
        const int wrow0 = row0 + wave * 32;
        const int qi = wrow0 + col;
        const bool valid = qi < p.Sq;
        const int qc = min(qi, p.Sq - 1);
        const int last_row = min(row0 + BM, p.Sq) - 1;
        const int wlast = min(wrow0 + 31, p.Sq - 1);

        int n_tiles = (p.Sk + BN - 1) / BN;
        if (p.causal) {
            const int hi = last_row + p.off;
            n_tiles = hi < 0 ? 0 : min(n_tiles, hi / BN + 1);
        }
        const int NB = n_tiles * 2;
        int NBw = NB;
        if (wrow0 >= p.Sq)
            NBw = 0;
        else if (p.causal) {
            const int wmax_lim = wlast + p.off;
            NBw = wmax_lim < 0 ? 0 : min(NB, wmax_lim / 32 + 1);
        }
        const int lim_lane = p.causal ? qi + p.off : 0x7fffffff;
        const int wmin_lim = p.causal ? wrow0 + p.off : 0x7fffffff;

        TL ld;
        ld.setup(p.k + ((long)b * p.Sk * p.Hkv + g) * D, p.v + ((long)b * p.Sk * p.Hkv + g) * D,
                 p.Hkv * D * 2, p.Sk);
        if (n_tiles > 0) ld.issue(lds, lds + TB, 0, wave, lane);
        if (n_tiles > 1) ld.issue(lds + STAGE, lds + STAGE + TB, BN, wave, lane);

        bf16x8_t qf[D / 16], dof[D / 16];
        const long rowoff = (((long)b * p.Sq + qc) * p.Hq + hq) * D;
        load_q<D>(qf, p.q + rowoff, half);
        load_q<D>(dof, p.dout + rowoff, half);
        const float lse2 = p.lse2[((long)b * p.Hq + hq) * p.Sq + qc];
        const float ndl = p.ndelta[((long)b * p.Hq + hq) * p.Sq + qc];
        wait_vmem();
        flip_q<D>(qf, p.flip);
        flip_q<D>(dof, 0u);

        f32x16_t dq[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) dq[db] = f32x16_t{};

        int st = 0;
        for (int t = 0; t < n_tiles; ++t) {
            char *stage = lds + st * STAGE;
            // tile t has landed (every wave's copies); tile t - 1's stage is free
            wait_vmem();
            __syncthreads();
            if (t + 2 < n_tiles) {
                const int s2 = st + 2 >= kPrefillStages ? st + 2 - kPrefillStages : st + 2;
                ld.issue(lds + s2 * STAGE, lds + s2 * STAGE + TB, (t + 2) * BN, wave, lane);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int j = 2 * t + kb;
                if (j >= NBw) continue;
                const char *Kblk = stage + kb * 32 * 2 * D;
                const char *Vblk = stage + TB + kb * 32 * 2 * D;
                f32x16_t s = BO::qk(Kblk, off, qf);
                const bool masked = (j * 32 + 32 > p.Sk) || (j * 32 + 31 > wmin_lim);
                if (masked) BO::mask(s, j * 32, half, p.Sk, lim_lane);
                const f32x16_t dp = BO::qk(Vblk, off, dof);
                float ds[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float pr = fast_exp2(fmaf(s[r], p.c, -lse2));
                    // masked keys score -inf: P = 0 also at scale 0 (-inf * 0 is NaN)
                    if (masked) pr = (s[r] == kNegInf) ? 0.0f : pr;
                    ds[r] = pr * (dp[r] + ndl);
                }
                bf16x8_t d0, d1;
                pack_halves(ds, d0, d1);
                bwd_accumulate<D>(Kblk, off, d0, d1, dq);
            }
            st = st + 1 == kPrefillStages ? 0 : st + 1;
        }
        __syncthreads();   // every wave is done with the LDS ring before the next item
        if (valid)
            store_rows<D, false>(dq, p.scale, half, p.dq, (((long)b * p.Sq + qi) * p.Hq + hq) * D);
    }
#endif
}

// dK, dV: one workgroup = NW waves x 32 keys of one (b, KV head); the Q and
// dO tiles of every query head of the group stream through a four-stage LDS
// ring (64 queries per tile, with their LSE and delta).  Per 32-query block
// n: S = Q K^T and dP = dO V^T (lane = key column, registers = queries),
// P = exp(S - LSE), dS = P (dP - delta), dV^T += dO^T P, dK^T += Q^T dS.
// With one wave per SIMD nothing else fills the matrix unit's idle cycles,
// so the block loop is software-pipelined: step n issues the S and dP MFMAs
// of block n + 1 and the accumulating MFMAs of block n - 1, and computes
// block n's P and dS on the VALU between them.  The three parts share no
// registers, so no MFMA waits for the softmax terms.  Tile u holds blocks 2u
// and 2u + 1.  Step 2u + 1 begins with the barrier that makes tile u + 1
// ready and tile u - 1's stage reusable (its last reader is the accumulation
// of block 2u - 1, in step 2u), then starts the copies of tile u + 3 into
// that stage.
// ---------------------------------------------------------------------------
constexpr int kBwdStages = 4;

template <int D>
struct BwdKeys {
    bf16x8_t kf[D / 16], vf[D / 16];   // this lane's key row of K and of V (B operands)
    f32x16_t dk[D / 32], dv[D / 32];   // dK^T and dV^T (lane = key column)
};

// One 32-query block in the ring: its Q rows and dO rows, and this lane's
// LSE * log2 e and -delta values (16 bytes at +32 g4: registers 4 g4 .. 4 g4 + 3).
struct BwdBlock {
    const char *q, *o;
    const char *lse, *ndl;
};

// -delta of a block's 16 rows of this lane in accumulator order: the initial
// value of its dP chain, which then yields dP - delta.
__device__ __forceinline__ f32x16_t bwd_ld_ndelta(const BwdBlock &b)
{
    f32x16_t d;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t *>(b.ndl + 32 * g4);
#pragma unroll
        for (int e = 0; e < 4; ++e) d[4 * g4 + e] = v[e];
    }
    return d;
}

// An S or dP MFMA chain's first step from a given accumulator (see mfma_s_first).
__device__ __forceinline__ void mfma_s_from(f32x16_t &d, bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
}

// The transposed operand of accumulating MFMA st of a block (see bwd_accumulate).
template <int D>
__device__ __forceinline__ bf16x8_t bwd_ld_tr(const char *X, const OperandOffsets<D> &off, int st)
{
    constexpr int DB = D / 32;
    const int t2 = st / DB, db = st % DB;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t *)(X + off.vofs(db, 0) + t2 * 16 * 2 * D));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t *)(X + off.vofs(db, 1) + t2 * 16 * 2 * D));
    const u32x2_t lw = __builtin_bit_cast(u32x2_t, lo);
    const u32x2_t hw = __builtin_bit_cast(u32x2_t, hi);
    return __builtin_bit_cast(bf16x8_t, (u32x4_t){lw[0], lw[1], hw[0], hw[1]});
}

// Step n of the dK/dV pipeline.  nx: block n + 1 (S and dP into sn, dpn);
// cu: block n (P and dS from s, dp into pn, dn); pv: block n - 1 (its P and
// dS in pp, dd accumulate into dV and dK; ACC = false: no such block).
// Slot st issues S k-step st, dV MFMA st, dP k-step st and dK MFMA st, with
// the slot's 16 / QS elements of P(n) and dS(n) spread between them, and
// copy(st), the slot's share of a later tile's HBM -> LDS copies; the
// operand reads run kBwdPrefetch slots ahead.  S and dP are inline-asm MFMAs
// with VGPR accumulators (the VALU reads them in the next step) and the K and
// V rows in AGPRs; the s_nop at the end of the step, with the slots after the
// last ones of each chain, covers their result latency before the next step
// (or a branch) may touch them, which the build's scan of the generated code
// checks.
constexpr int kBwdPrefetch = 2;

template <int D, bool ACC, class CP>
__device__ __forceinline__ void bwd_kv_step(BwdKeys<D> &w, const OperandOffsets<D> &off,
                                            const BwdBlock &nx, const BwdBlock &cu,
                                            const BwdBlock &pv, float c,
                                            const f32x16_t &s, const f32x16_t &dp,
                                            f32x16_t &sn, f32x16_t &dpn, const bf16x8_t (&pp)[2],
                                            const bf16x8_t (&dd)[2], bf16x8_t (&pn)[2],
                                            bf16x8_t (&dn)[2], CP &&copy)
{
    constexpr int QS = D / 16, DB = D / 32, EPS = 16 / QS;
    constexpr int PF = kBwdPrefetch < QS ? kBwdPrefetch : QS;
    bf16x8_t qa[QS], oa[QS], va[QS], ka[QS];
    f32x4_t lv[4];
    u32x4_t pw[2], dw[2];
    // the reads of slot i, in the order the slots consume them (LDS reads
    // complete in order); the LSE of a group of 4 rows comes with the slot
    // that first needs it, block n + 1's -delta (the dP chain's start) with
    // slot 0
    f32x16_t nd;
    auto rd = [&](int i) {
        qa[i] = *reinterpret_cast<const bf16x8_t *>(nx.q + off.kofs(i));
        if (i == 0) nd = bwd_ld_ndelta(nx);
        if ((i * EPS) % 4 == 0) {
            const int g4 = i * EPS / 4;
            lv[g4] = *reinterpret_cast<const f32x4_t *>(cu.lse + 32 * g4);
        }
        if (ACC) va[i] = bwd_ld_tr<D>(pv.o, off, i);
        oa[i] = *reinterpret_cast<const bf16x8_t *>(nx.o + off.kofs(i));
        if (ACC) ka[i] = bwd_ld_tr<D>(pv.q, off, i);
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) rd(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < QS; ++st) {
        const int t2 = st / DB, db = st % DB;
        float x[EPS], y[EPS];
        if (st == 0) mfma_s_first(sn, qa[st], w.kf[st]);
        else mfma_s_next(sn, qa[st], w.kf[st]);
        __builtin_amdgcn_sched_barrier(0);
        if (st + PF < QS) rd(st + PF);
#pragma unroll
        for (int i = 0; i < EPS; ++i) {
            const int r = st * EPS + i, g4 = r / 4, e = r % 4;
            x[i] = fmaf(s[r], c, -lv[g4][e]);
        }
#pragma unroll
        for (int i = 0; i < EPS / 2; ++i) {
            y[i] = fast_exp2(x[i]);
            keep(y[i]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (ACC) w.dv[db] = mfma32(va[st], pp[t2], w.dv[db]);
        __builtin_amdgcn_sched_barrier(0);
        copy(st);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = EPS / 2; i < EPS; ++i) {
            y[i] = fast_exp2(x[i]);
            keep(y[i]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (st == 0) mfma_s_from(dpn, oa[st], w.vf[st], nd);
        else mfma_s_next(dpn, oa[st], w.vf[st]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < EPS; i += 2) {
            const int r = st * EPS + i;
            const float d0 = y[i] * dp[r];       // dp: dP - delta
            const float d1 = y[i + 1] * dp[r + 1];
            const int wi = r / 2;   // bf16 pair: word wi % 4 of half wi / 4
            pw[wi / 4][wi % 4] = pack_bf16(y[i], y[i + 1]);
            dw[wi / 4][wi % 4] = pack_bf16(d0, d1);
            keep(pw[wi / 4][wi % 4]);
            keep(dw[wi / 4][wi % 4]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (ACC) w.dk[db] = mfma32(ka[st], dd[t2], w.dk[db]);
        __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_nop 7" : "+v"(sn), "+v"(dpn)::"memory");
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        pn[h] = __builtin_bit_cast(bf16x8_t, pw[h]);
        dn[h] = __builtin_bit_cast(bf16x8_t, dw[h]);
    }
}

// Causal blocks that cross the diagonal, between steps: element r of the
// lane (query base + 8 (r / 4) + r % 4) is allowed only if that offset is at
// least lo; the others score -inf, so that P = 0 there (c > 0).  Rows past
// the last query need no mask: their Q and dO rows, LSE and delta read as
// zero, so that P = 1 and dS = 0 there, and both accumulating products add
// exact zeros.  Keys past the last key need none either: a lane's values
// only reach its own columns of dK and dV, which are not stored.
__device__ __forceinline__ void bwd_mask_rows(f32x16_t &s, int lo)
{
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = (8 * (r >> 2) + (r & 3) < lo) ? kNegInf : s[r];
}

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1)))
fa_bwd_dkdv_kernel(const BwdParams p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int BQ = 64;
    constexpr int BK = 32 * NW;
    using TL = TileLoader<D, BQ, NW>;
    constexpr int TB = TL::TILE_BYTES;
    constexpr int STAGE = 2 * TB + 1024;   // Q tile, dO tile, LSE * log2e, delta
    constexpr int LPU = 2 * TL::PER_WAVE;  // Q and dO row copies per wave and tile
    static_assert(LPU + 2 <= 15, "vmcnt immediate");
    __shared__ __attribute__((aligned(1024))) char lds[kBwdStages * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;
    OperandOffsets<D> off;
    off.init(lane);

    // (b, g) pairs in 8 residue classes, one per XCD, as in fa_bwd_dq_kernel:
    // the key blocks of a KV head stream the same Q and dO tiles through one L2
    const int BG = p.B * p.Hkv;
    const int ND = (BG % 8 == 0 && gridDim.x % 8 == 0) ? 8 : 1;
    const int x = blockIdx.x % ND;
    const int jw = blockIdx.x / ND;
    const int Gx = gridDim.x / ND;
    const int N = (BG / ND) * p.n_blocks;
    const int ntq_all = (p.Sq + BQ - 1) / BQ;
    // byte offset of each of this lane's Q / dO row copies within a tile
    // (row stride Hq * D * 2, 16-byte chunks placed by the tile swizzle)
    const int qstride = p.Hq * D * 2;
    int loff[TL::PER_WAVE];
#pragma unroll
    for (int i = 0; i < TL::PER_WAVE; ++i) {
        const int row = (i * NW + wave) * TL::RPI + lane / TL::CPR;
        loff[i] = row * qstride + (((lane % TL::CPR) ^ swz<D>(row)) * 16);
    }
    // scale 0: S is 0 for every pair, which zero K rows give exactly; with
    // c = 1 the diagonal mask's -inf then still gives P = 0
    const bool zero_scale = p.c == 0.0f;
    const float c = zero_scale ? 1.0f : p.c;
    for (int it = 0; it * Gx < N; ++it) {
        const int li = it * Gx + ((it & 1) ? (Gx - 1 - jw) : jw);
        if (li >= N) continue;
        // (b, g) by (b, g), each one's first (causal: longest) key blocks first
        const int bg = (li / p.n_blocks) * ND + x;
        const int kblk = li % p.n_blocks;
        const int b = bg / p.Hkv;
        const int g = bg % p.Hkv;
        const int k0 = kblk * BK;                 // first key of the workgroup
        const int kw0 = k0 + wave * 32;           // first key of the wave
        const int kj = kw0 + col;                 // this lane's key
        const bool kvalid = kj < p.Sk;
        const int kc = min(kj, p.Sk - 1);
        // causal: query i sees key j iff j <= i + off, i.e. i >= j - off
        const int t0 = p.causal ? max(0, k0 - p.off) / BQ : 0;
        const int ntq = max(0, ntq_all - t0);
        const int n_units = ntq * p.group;        // (head, query tile) pairs

        // copies of tile u (query head g * group + u / ntq, query tile
        // t0 + u % ntq), in LPU + 2 copy instructions per wave: the Q and dO
        // rows in PER_WAVE pairs, then the LSE and delta vectors (wave 0; the
        // other waves copy an empty range into the stage's spare bytes, so
        // that every wave counts as many copies per tile).  Tiles past the
        // last one are copied the same way from empty ranges: they fill a
        // free stage with zeros and keep the count per tile fixed.
        int cp_h = 0, cp_t = 0;   // head within the group and tile of the next tile to copy
        u32x4_t cq, co, cl, cd;
        int ctoff = 0, cstage = 0;
        auto copy_begin = [&]() {
            const bool real = cp_h < p.group;
            const int hq = g * p.group + (real ? cp_h : 0);
            const int t = t0 + cp_t;
            const long hbase = ((long)b * p.Sq * p.Hq + hq) * D;
            const uint32_t nbytes = real ? (uint32_t)((p.Sq - 1) * qstride + D * 2) : 0u;
            cq = raw_desc(p.q + hbase, nbytes);
            co = raw_desc(p.dout + hbase, nbytes);
            const long vb = ((long)b * p.Hq + hq) * p.Sq + (long)t * BQ;
            const uint32_t nb = (real && wave == 0) ? (uint32_t)((p.Sq - t * BQ) * 4) : 0u;
            cl = raw_desc(p.lse2 + vb, nb);
            cd = raw_desc(p.ndelta + vb, nb);
            ctoff = t * BQ * qstride;
            if (++cp_t == ntq) {
                cp_t = 0;
                ++cp_h;
            }
        };
        auto copy_part = [&](int i) {
            char *dst = lds + cstage * STAGE;
            if (i < TL::PER_WAVE) {
                const int q = i * NW + wave;
                lds_dma16_pair(dst + q * 1024, dst + TB + q * 1024, ctoff + loff[i], cq, co);
            } else if (i == TL::PER_WAVE) {
                const int spare = wave == 0 ? 0 : 256;
                lds_dma4_pair(dst + 2 * TB + spare, dst + 2 * TB + 512 + spare, lane * 4, cl, cd);
            }
        };
        auto copy_tile = [&](int u) {
            cstage = u % kBwdStages;
            copy_begin();
#pragma unroll
            for (int i = 0; i <= TL::PER_WAVE; ++i) copy_part(i);
        };
        auto no_copy = [](int) {};
        auto block_of = [&](int u, int qb) {
            const char *stg = lds + (u % kBwdStages) * STAGE;
            return BwdBlock{stg + qb * 32 * 2 * D, stg + TB + qb * 32 * 2 * D,
                            stg + 2 * TB + qb * 128 + 16 * half,
                            stg + 2 * TB + 512 + qb * 128 + 16 * half};
        };
        // whether block qb of tile u crosses the causal diagonal for this
        // wave, and the lane's smallest allowed row offset there
        auto mask_of = [&](int u, int qb, int &lo) {
            const int q0 = (t0 + u % ntq) * BQ + qb * 32;
            lo = kj - p.off - (q0 + 4 * half);
            return p.causal && kw0 + 31 > q0 + p.off;
        };

        if (n_units > 0) copy_tile(0);
        BwdKeys<D> w;
        load_q<D>(w.kf, p.k + (((long)b * p.Sk + kc) * p.Hkv + g) * D, half);
        load_q<D>(w.vf, p.v + (((long)b * p.Sk + kc) * p.Hkv + g) * D, half);
        wait_vmem();
        if (zero_scale) {
#pragma unroll
            for (int st = 0; st < D / 16; ++st) w.kf[st] = bf16x8_t{};
        }
        flip_q<D>(w.kf, p.flip);
        flip_q<D>(w.vf, 0u);
        // the K and V rows are only ever B operands of inline-asm MFMAs:
        // moved to AGPRs here, once, not before each MFMA
#pragma unroll
        for (int st = 0; st < D / 16; ++st) asm volatile("" : "+a"(w.kf[st]), "+a"(w.vf[st]));
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            w.dk[db] = f32x16_t{};
            w.dv[db] = f32x16_t{};
        }
        __syncthreads();   // tile 0 is in LDS (every wave's copies)

        if (n_units > 0) {
            copy_tile(1);
            copy_tile(2);
            copy_begin();   // tile 3's descriptors, for step 1
            f32x16_t sx, dpx, sy, dpy;             // S, dP of the even / odd block
            bf16x8_t px[2], dx[2], py[2], dy[2];   // their P and dS (B operands)
            int lo;
            {
                // S(0), dP(0); step 0: S(1), P(0)
                const BwdBlock c0 = block_of(0, 0), c1 = block_of(0, 1);
#pragma unroll
                for (int st = 0; st < D / 16; ++st) {
                    const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(c0.q + off.kofs(st));
                    const bf16x8_t o = *reinterpret_cast<const bf16x8_t *>(c0.o + off.kofs(st));
                    if (st == 0) {
                        mfma_s_first(sx, a, w.kf[st]);
                        mfma_s_from(dpx, o, w.vf[st], bwd_ld_ndelta(c0));
                    } else {
                        mfma_s_next(sx, a, w.kf[st]);
                        mfma_s_next(dpx, o, w.vf[st]);
                    }
                }
                mfma_s_drain(sx, dpx);
                if (mask_of(0, 0, lo)) bwd_mask_rows(sx, lo);
                bwd_kv_step<D, false>(w, off, c1, c0, c0, c, sx, dpx, sy, dpy, py, dy, px, dx,
                                      no_copy);
            }
            for (int u = 0; u < n_units; ++u) {
                const BwdBlock c0 = block_of(u, 0), c1 = block_of(u, 1);
                // step 2u + 1: S(2u + 2) from tile u + 1 (zeros past the last
                // tile: a dead S), P(2u + 1), accumulation of block 2u, and
                // the copies of tile u + 3 into tile u - 1's stage.  Tile
                // u + 2's copies may stay in flight.
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(0x0F70 | (LPU + 2));
                pp_barrier();
                cstage = (u + 3) % kBwdStages;
                if (mask_of(u, 1, lo)) bwd_mask_rows(sy, lo);
                bwd_kv_step<D, true>(w, off, block_of(u + 1, 0), c1, c0, c, sy, dpy, sx, dpx, px,
                                     dx, py, dy, copy_part);
                if (u + 1 < n_units) {
                    // step 2u + 2: S(2u + 3), P(2u + 2), accumulation of block
                    // 2u + 1, and the descriptors of tile u + 4's copies
                    const BwdBlock n0 = block_of(u + 1, 0), n1 = block_of(u + 1, 1);
                    if (mask_of(u + 1, 0, lo)) bwd_mask_rows(sx, lo);
                    bwd_kv_step<D, true>(w, off, n1, n0, c1, c, sx, dpx, sy, dpy, py, dy, px, dx,
                                         [&](int st) {
                                             if (st == 1) copy_begin();
                                         });
                }
            }
            const BwdBlock last = block_of(n_units - 1, 1);
            bwd_accumulate<D>(last.o, off, py[0], py[1], w.dv);
            bwd_accumulate<D>(last.q, off, dy[0], dy[1], w.dk);
        }
        __syncthreads();   // every wave is done with the ring before the next item
        if (kvalid) {
            const long kb_off = (((long)b * p.Sk + kj) * p.Hkv + g) * D;
            store_rows<D, false>(w.dk, p.scale, half, p.dk, kb_off);
            store_rows<D, false>(w.dv, 1.0f, half, p.dv, kb_off);
        }
    }
#endif
}
// ---------------------------------------------------------------------------
// Wide prefill: one wave per SIMD, 64 query rows per wave (column blocks
// r = 0, 1 of 32 rows), so that each K and V operand read from LDS feeds two
// MFMAs -- half the LDS reads per flop of the kernel above.  With one wave
// per SIMD no other wave fills the matrix unit's shadow, so the block loop is
// software-pipelined by hand: block j issues, step by step, the MFMAs of
// S(j+1) = K Q^T and of O += V P(j-1), and between them the VALU work that
// turns S(j) into P(j).  The reference max is the exact row max of the first
// key block; after that it moves only when a block's exact P sum (which the
// LSE needs anyway) exceeds kWideOverflow in some lane -- that block is then
// redone against its exact row max.  P therefore stays below 2^64: bf16 and
// fp32 carry the same relative precision at any magnitude, and the sums stay
// far from fp32 overflow (O and the row sums grow to at most keys * 2^64 *
// max|v|, below 2^127 for any key count under 2^50 with |v| < 2^13).  The
// threshold only has to catch exponents near overflow (an exp2 of 128 or
// more is inf, which the test also catches); a low one would redo a block
// each time a row's running max climbs, as it does on rows with large
// scores.
// LDS: the three K tiles first, then the three V tiles; the V operand offsets
// carry the distance between the two, so that the stage and block parts of
// every LDS address are compile-time immediates.
// ---------------------------------------------------------------------------
constexpr float kWideOverflow = 18446744073709551616.0f;   // 2^64
// Operand reads of the fast block run this many steps ahead of their MFMAs.
constexpr int kWidePrefetch = 2;
// Slots of a pipelined step whose operands are read ahead (the first ones
// at the end of the step before).
constexpr int kPipePF = 2;

template <int D>
struct WideRows {
    static constexpr int QS = D / 16;
    static constexpr int DB = D / 32;
    bf16x8_t qf[2][QS];
    f32x16_t o[2][DB];
    f32x16_t s[2];        // S^T of block j, to be turned into P(j)
    bf16x8_t pp[2][2];    // P(j - 1), waiting for its P V
    f32x4_t l_acc[2];     // element 0: row sum of the rounded P (whole row)
    float m_ref[2];       // reference max (score units)
    float mc[2];          // c * m_ref, 0 while m_ref = -inf
    float l_run[2];       // exact row sum (this lane half)
    int lim[2];           // causal limit of this lane's row in column block r
    bf16x8_t sel;         // row-sum selector operand
    int NBw;              // blocks this wave has work on (a prefix of the tile walk)
    int wmin_lim;         // smallest causal limit of the wave's rows
    int key_end;
    int half;
    float c;

    __device__ __forceinline__ bool needs_mask(int j) const
    {
        return (j * 32 + 32 > key_end) || (j * 32 + 31 > wmin_lim);
    }
};

template <int D>
__device__ __forceinline__ bf16x8_t wide_ld_k(const char *Kblk, const OperandOffsets<D> &off, int st)
{
    return *reinterpret_cast<const bf16x8_t *>(Kblk + off.kofs(st));
}

// A operand of PV step ps (16 keys x 32 head dims) of the block at Vblk.
template <int D>
__device__ __forceinline__ bf16x8_t wide_ld_v(const char *Vblk, const OperandOffsets<D> &off, int ps)
{
    constexpr int DB = D / 32;
    const int t2 = ps / DB, db = ps % DB;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t *)(Vblk + off.vofs(db, 0) + t2 * 16 * 2 * D));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t *)(Vblk + off.vofs(db, 1) + t2 * 16 * 2 * D));
    const u32x2_t lw = __builtin_bit_cast(u32x2_t, lo);
    const u32x2_t hw = __builtin_bit_cast(u32x2_t, hi);
    return __builtin_bit_cast(bf16x8_t, (u32x4_t){lw[0], lw[1], hw[0], hw[1]});
}

// S^T of one 32-key block (K rows at Kblk) for both column blocks.  All K
// fragments are read first: the MFMAs are volatile asm, which the compiler
// does not move loads across, so a read inside the loop would cost one LDS
// round trip per k-step.
template <int D>
__device__ __forceinline__ void wide_qk(const char *Kblk, const OperandOffsets<D> &off,
                                        const bf16x8_t (&qf)[2][D / 16], f32x16_t (&s)[2])
{
    bf16x8_t ka[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st) ka[st] = wide_ld_k<D>(Kblk, off, st);
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
        const bf16x8_t a = ka[st];
        if (st == 0) {
            mfma_s_first(s[0], a, qf[0][0]);
            mfma_s_first(s[1], a, qf[1][0]);
        } else {
            mfma_s_next(s[0], a, qf[0][st]);
            mfma_s_next(s[1], a, qf[1][st]);
        }
    }
    mfma_s_drain(s[0], s[1]);
}

// P of key pair q (registers 2q, 2q+1) of one column block: exp2(c*s - mc),
// packed to bf16 into w[q / 4][q % 4]; la adds the exact values.
template <bool MASK>
__device__ __forceinline__ void wide_pair(const f32x16_t &s, int q, float c, float mc,
                                          u32x4_t (&w)[2], float &la)
{
    float a = fast_exp2(fmaf(s[2 * q], c, -mc));
    float b = fast_exp2(fmaf(s[2 * q + 1], c, -mc));
    if (MASK) {
        a = (s[2 * q] == kNegInf) ? 0.0f : a;
        b = (s[2 * q + 1] == kNegInf) ? 0.0f : b;
    }
    w[q >> 2][q & 3] = pack_bf16(a, b);
    la += a + b;
}


// End of block j: where P(j) overflowed, redo it against the exact row max;
// then P(j) becomes the pending P and S(j+1) the next S.
template <int D, bool MASK>
__device__ __forceinline__ void wide_settle(WideRows<D> &w, const f32x16_t (&sn)[2],
                                            u32x4_t (&pw)[2][2], float (&la)[2], int key0 = -1)
{
    constexpr int DB = D / 32;
    // !(x <= T) is also true for inf and NaN
    const bool big = !(la[0] <= kWideOverflow) || !(la[1] <= kWideOverflow);
    if (__any(big)) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            // a masked fast block masked only its P: mask S(j) for the redo
            if (MASK && key0 >= 0) BlockOps<D>::mask(w.s[r], key0, w.half, w.key_end, w.lim[r]);
            float mx = kNegInf;
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, w.s[r][e]);
            mx = max_halves(mx);
            const float m_new = fmaxf(w.m_ref[r], mx);
            const float alpha =
                (w.m_ref[r] == kNegInf) ? 0.0f : fast_exp2((w.m_ref[r] - m_new) * w.c);
            w.l_run[r] *= alpha;
            w.l_acc[r][0] *= alpha;
            // one accumulator at a time: O lives in AGPRs, and rescaling it
            // all at once would need 64 VGPRs of temporaries in this loop
#pragma unroll
            for (int db = 0; db < DB; ++db) {
#pragma unroll
                for (int e = 0; e < 16; ++e) w.o[r][db][e] *= alpha;
                __builtin_amdgcn_sched_barrier(0);
            }
            w.m_ref[r] = m_new;
            w.mc[r] = (m_new == kNegInf) ? 0.0f : m_new * w.c;
            la[r] = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) wide_pair<MASK>(w.s[r], q, w.c, w.mc[r], pw[r], la[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        w.l_run[r] += la[r];
        w.pp[r][0] = __builtin_bit_cast(bf16x8_t, pw[r][0]);
        w.pp[r][1] = __builtin_bit_cast(bf16x8_t, pw[r][1]);
        w.s[r] = sn[r];
    }
}

// Block j with every piece live and no mask: S(j+1) from the K block at Kn,
// O += V P(j-1) from the V block at Vp, P(j) from S(j).  Step st issues the
// operand reads of step st + kWidePrefetch, the two S MFMAs of k-step st and
// the two P V MFMAs of PV step st, and between consecutive MFMAs one quarter
// of the step's share of P(j), placed so that no value is consumed in the
// MFMA shadow that produces it (one wave per SIMD: a dependent instruction
// right behind a transcendental would stall the wave, and the next MFMA with
// it).  The order is fixed with scheduling fences (the S MFMAs are inline
// asm, which the scheduler's grouping does not recognise).
//
// MASK: block j (keys from key0) may cross the causal diagonal or the key
// end; masked keys get exponent -inf, so P is 0 there for any scale.
template <int D, bool MASK = false>
__device__ __forceinline__ void wide_block_fast(const char *Kn, const char *Vp,
                                                const OperandOffsets<D> &off, WideRows<D> &w,
                                                int key0 = 0)
{
    constexpr int QS = D / 16, DB = D / 32, PPS = 8 / QS;
    constexpr int PF = kWidePrefetch < QS ? kWidePrefetch : QS;
    // largest allowed key offset from this lane half's first key (as in
    // BlockOps::mask)
    int last[2] = {0, 0};
    if (MASK) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
            last[r] = min(w.lim[r], w.key_end - 1) - (key0 + 4 * w.half);
    }
    f32x16_t sn[2];
    u32x4_t pw[2][2];
    float la[2] = {-0.0f, -0.0f};   // -0 + x is x: the first add folds away
    bf16x8_t kr[QS], vr[QS];
    // in the order the steps consume them, so that the first MFMA waits for
    // one LDS read only (LDS reads complete in order)
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        kr[i] = wide_ld_k<D>(Kn, off, i);
        __builtin_amdgcn_sched_barrier(0);
        vr[i] = wide_ld_v<D>(Vp, off, i);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int st = 0; st < QS; ++st) {
        const bool pf = st + PF < QS;
        const int t2 = st / DB, db = st % DB;
        // the step's VALU work, spread over the four MFMA shadows so that no
        // result is read in the shadow it is produced in: both column blocks'
        // exponent arguments; the exps, r = 0 first; then per column block
        // the bf16 pairs and the exact sums
        float xa[2][PPS][2], ya[2][PPS][2];
        if (st == 0)
            mfma_s_first(sn[0], kr[st], w.qf[0][st]);
        else
            mfma_s_next(sn[0], kr[st], w.qf[0][st]);
        __builtin_amdgcn_sched_barrier(0);
        if (pf) kr[st + PF] = wide_ld_k<D>(Kn, off, st + PF);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int p = 0; p < PPS; ++p) {
                const int q = st * PPS + p;
                xa[r][p][0] = fmaf(w.s[r][2 * q], w.c, -w.mc[r]);
                xa[r][p][1] = fmaf(w.s[r][2 * q + 1], w.c, -w.mc[r]);
                if (MASK) {
                    const int e0 = 2 * q, e1 = 2 * q + 1;
                    xa[r][p][0] = (8 * (e0 >> 2) + (e0 & 3) > last[r]) ? kNegInf : xa[r][p][0];
                    xa[r][p][1] = (8 * (e1 >> 2) + (e1 & 3) > last[r]) ? kNegInf : xa[r][p][1];
                }
            }
#pragma unroll
        for (int p = 0; p < PPS; ++p) {
            ya[0][p][0] = fast_exp2(xa[0][p][0]);
            keep(ya[0][p][0]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (st == 0)
            mfma_s_first(sn[1], kr[st], w.qf[1][st]);
        else
            mfma_s_next(sn[1], kr[st], w.qf[1][st]);
        __builtin_amdgcn_sched_barrier(0);
        if (pf) vr[st + PF] = wide_ld_v<D>(Vp, off, st + PF);
#pragma unroll
        for (int p = 0; p < PPS; ++p) {
            ya[0][p][1] = fast_exp2(xa[0][p][1]);
            ya[1][p][0] = fast_exp2(xa[1][p][0]);
            keep(ya[0][p][1]);
            keep(ya[1][p][0]);
        }
        __builtin_amdgcn_sched_barrier(0);
        w.o[0][db] = mfma32(vr[st], w.pp[0][t2], w.o[0][db]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < PPS; ++p) {
            const int q = st * PPS + p;
            ya[1][p][1] = fast_exp2(xa[1][p][1]);
            keep(ya[1][p][1]);
            pw[0][q >> 2][q & 3] = pack_bf16(ya[0][p][0], ya[0][p][1]);
            la[0] += ya[0][p][0] + ya[0][p][1];
            keep(pw[0][q >> 2][q & 3]);
        }
        __builtin_amdgcn_sched_barrier(0);
        w.o[1][db] = mfma32(vr[st], w.pp[1][t2], w.o[1][db]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < PPS; ++p) {
            const int q = st * PPS + p;
            pw[1][q >> 2][q & 3] = pack_bf16(ya[1][p][0], ya[1][p][1]);
            la[1] += ya[1][p][0] + ya[1][p][1];
            keep(pw[1][q >> 2][q & 3]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (st == QS - 2) {
            w.l_acc[0] = mfma16(w.sel, w.pp[0][0], w.l_acc[0]);
            w.l_acc[0] = mfma16(w.sel, w.pp[0][1], w.l_acc[0]);
        }
        if (st == QS - 1) {
            w.l_acc[1] = mfma16(w.sel, w.pp[1][0], w.l_acc[1]);
            w.l_acc[1] = mfma16(w.sel, w.pp[1][1], w.l_acc[1]);
        }
    }
    mfma_s_fence(sn[0], sn[1]);
    wide_settle<D, MASK>(w, sn, pw, la, MASK ? key0 : -1);
}

// Block j in general: any of S(j+1), P V(j-1), P(j) may be absent for this
// wave, and keys past key_end or the causal limit are masked.
template <int D>
__device__ __forceinline__ void wide_block_general(const char *Kn, const char *Vp, int j,
                                                   const OperandOffsets<D> &off, WideRows<D> &w)
{
    constexpr int QS = D / 16, DB = D / 32;
    const bool live = j < w.NBw;
    const bool live_next = j + 1 < w.NBw;
    const bool live_prev = j >= 1 && j - 1 < w.NBw;
    f32x16_t sn[2] = {f32x16_t{}, f32x16_t{}};
    if (live_next) wide_qk<D>(Kn, off, w.qf, sn);
    if (live_prev) {
#pragma unroll
        for (int ps = 0; ps < QS; ++ps) {
            const bf16x8_t a = wide_ld_v<D>(Vp, off, ps);
            const int t2 = ps / DB, db = ps % DB;
            w.o[0][db] = mfma32(a, w.pp[0][t2], w.o[0][db]);
            w.o[1][db] = mfma32(a, w.pp[1][t2], w.o[1][db]);
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            w.l_acc[r] = mfma16(w.sel, w.pp[r][0], w.l_acc[r]);
            w.l_acc[r] = mfma16(w.sel, w.pp[r][1], w.l_acc[r]);
        }
    }
    if (live) {
        u32x4_t pw[2][2];
        float la[2] = {0.0f, 0.0f};
        const bool m = w.needs_mask(j);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            if (m) BlockOps<D>::mask(w.s[r], j * 32, w.half, w.key_end, w.lim[r]);
#pragma unroll
            for (int q = 0; q < 8; ++q) wide_pair<true>(w.s[r], q, w.c, w.mc[r], pw[r], la[r]);
        }
        wide_settle<D, true>(w, sn, pw, la);
    } else {
        w.s[0] = sn[0];
        w.s[1] = sn[1];
    }
}

// The blocks of tile t (LDS stage `stage`); `next` holds tile t + 1 and
// `prev` tile t - 1, whose stage receives tile t + 2 once the barrier in the
// tile's last block shows every wave is done with it.  Needs BN >= 64: the
// P V of a tile's first block reads the last block of tile t - 1, which must
// still be in place.
template <int D, int BN, int NW, bool FAST, bool MASK = false>
__device__ __forceinline__ void wide_tile(int t, int n_tiles, char *stage, char *next, char *prev,
                                          const TileLoader<D, BN, NW> &ld, int wave, int lane,
                                          const OperandOffsets<D> &off, WideRows<D> &w)
{
    constexpr int KB = BN / 32;
    constexpr int TB = TileLoader<D, BN, NW>::TILE_BYTES;
    static_assert(KB >= 2, "the wide prefill needs at least two key blocks per tile");
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const char *Kn = (kb == KB - 1) ? next : stage + (kb + 1) * 32 * 2 * D;
        // V of the previous block; its offsets add the K-to-V distance
        const char *Vp = (kb == 0) ? prev + (KB - 1) * 32 * 2 * D : stage + (kb - 1) * 32 * 2 * D;
        // (a fast tile that is not masked always has a next tile)
        if (kb == KB - 1 && t + 1 < n_tiles) {
            wait_vmem();       // this wave's copies of tile t + 1 are in LDS
            __syncthreads();   // ... and every wave's; tile t - 1 is released
            if (t + 2 < n_tiles)
                ld.issue(prev, prev + kPrefillStages * TB, (t + 2) * BN, wave, lane);
        }
        if (FAST)
            wide_block_fast<D, MASK>(Kn, Vp, off, w, (t * KB + kb) * 32);
        else
            wide_block_general<D>(Kn, Vp, t * KB + kb, off, w);
    }
}

// A tile takes the fast body when t >= 1 (its first block has a pending
// P V), its blocks and the block after it are live for this wave and none of
// its blocks needs a mask.  Liveness and masking are monotone in the block
// index, so the fast tiles of a wave form one range [1, t_end).  (The block
// after it being live implies t + 1 < n_tiles: the fast body always takes
// the tile-boundary barrier.)
template <int KB>
__device__ __forceinline__ bool wide_fast_ok(int t, int NBw, int key_end, int wmin_lim)
{
    const int jl = t * KB + KB - 1;   // the tile's last block
    return t >= 1 && jl + 1 < NBw && jl * 32 + 32 <= key_end && jl * 32 + 31 <= wmin_lim;
}

// The tile after the fast range takes the masked fast body when t >= 1 and
// all its blocks are live for this wave (the diagonal or the key end cuts
// it).  Its last block's S(j+1) is computed even when block j+1 is dead (from
// whatever the next stage holds) and then never used.
template <int KB>
__device__ __forceinline__ bool wide_masked_ok(int t, int NBw)
{
    return t >= 1 && t * KB + KB - 1 < NBw;
}

// One work item of the 64-row kernel: 256 query rows of one (b, hq).
struct WideItem {
    int b, hq, g;
    int wrow0;     // this wave's first query row
    int n_tiles;   // key tiles the workgroup walks
    int NBw;       // key blocks this wave has work on (a prefix of the walk)
};

// Item `it` of this workgroup, if it has one.  The snake over `it` balances
// the causal lengths; rank-major walks all heads' longest blocks first,
// head-major all blocks of one head before the next (more workgroups of an
// XCD then stream the same K/V at once).  Items past the end only occur on
// the last trip, so the valid items of a workgroup are a prefix of `it`.
__device__ __forceinline__ bool wide_item(const Params &p, int it, int Gx, int jw, int x, int Nx,
                                          int BHx, int ND, int BM, int BN, int wave, WideItem &I)
{
    if (it * Gx >= Nx) return false;
    const int li = it * Gx + ((it & 1) ? (Gx - 1 - jw) : jw);
    if (li >= Nx) return false;
    const int rank = p.head_major ? li % p.n_mblocks : li / BHx;
    const int bh = (p.head_major ? li / p.n_mblocks : li % BHx) * ND + x;
    const int mb = p.causal ? (p.n_mblocks - 1 - rank) : rank;
    I.b = bh / p.Hq;
    I.hq = bh % p.Hq;
    I.g = I.hq / p.group;
    const int row0 = mb * BM;
    I.wrow0 = row0 + wave * 64;
    const int last_row = min(row0 + BM, p.Sq) - 1;
    const int wlast = min(I.wrow0 + 63, p.Sq - 1);
    int n_tiles = (p.Sk + BN - 1) / BN;
    if (p.causal) {
        const int hi = last_row + p.off;
        n_tiles = hi < 0 ? 0 : min(n_tiles, hi / BN + 1);
    }
    I.n_tiles = n_tiles;
    const int NB = n_tiles * (BN / 32);
    if (I.wrow0 >= p.Sq)
        I.NBw = 0;
    else if (p.causal) {
        const int wmax_lim = wlast + p.off;
        I.NBw = wmax_lim < 0 ? 0 : min(NB, wmax_lim / 32 + 1);
    } else
        I.NBw = NB;
    return true;
}

// The item's first two tiles' copies, then its Q loads (raw, into qf):
// one memory round trip for all, waited for at the item's start.
template <int D, int BN, int NW>
__device__ __forceinline__ void wide_item_issue(const Params &p, const WideItem &I,
                                                TileLoader<D, BN, NW> &ld, char *lds, int VOFF,
                                                int TB, int wave, int lane, int half, int col,
                                                bf16x8_t (&qf)[2][D / 16])
{
    ld.setup(p.k + ((long)I.b * p.Sk * p.Hkv + I.g) * D, p.v + ((long)I.b * p.Sk * p.Hkv + I.g) * D,
             p.Hkv * D * 2, p.Sk);
    if (I.n_tiles > 0) ld.issue(lds, lds + VOFF, 0, wave, lane);
    // D = 128: tile 1's first key behind an opaque value, so that its
    // offsets are formed here from the per-lane parts tile 0 uses instead of
    // being precomputed for the whole kernel (the register allocator spilled
    // those, and each reload between copies waited for every copy before it;
    // D = 64 has registers to spare and measured faster without this)
    int k1 = BN;
    if constexpr (D >= 128) asm volatile("" : "+s"(k1));
    if (I.n_tiles > 1) ld.issue(lds + TB, lds + TB + VOFF, k1, wave, lane);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int qi = min(I.wrow0 + 32 * r + col, p.Sq - 1);
        load_q<D>(qf[r], p.q + (((long)I.b * p.Sq + qi) * p.Hq + I.hq) * D, half);
    }
}

template <int D, int BN, int NW, bool OUT_F32>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1)))
fa_prefill_wide_kernel(const Params p)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    constexpr int BM = 64 * NW;
    constexpr int KB = BN / 32;
    constexpr int QS = D / 16;
    using TL = TileLoader<D, BN, NW>;
    constexpr int TB = TL::TILE_BYTES;
    constexpr int VOFF = kPrefillStages * TB;   // V tile s sits at K tile s + VOFF

    __shared__ __attribute__((aligned(1024))) char lds[2 * kPrefillStages * TB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;

    OperandOffsets<D> off;
    off.init(lane);
#pragma unroll
    for (int db = 0; db < OperandOffsets<D>::NV; ++db)
#pragma unroll
        for (int sec = 0; sec < 2; ++sec) {
            off.v[db][sec] += VOFF;
            // keep the bias inside the register: folded back into the
            // immediates it would overflow their 16 bits
            asm volatile("" : "+v"(off.v[db][sec]));
        }

    const int BH = p.B * p.Hq;
    const int ND = p.domains;
    const int x = blockIdx.x % ND;
    const int jw = blockIdx.x / ND;
    const int Gx = gridDim.x / ND;
    const int BHx = BH / ND;
    const int Nx = BHx * p.n_mblocks;

    // Items are software-pipelined: the next item's first two K/V tiles and
    // its Q are requested as soon as the LDS ring is free, before this
    // item's epilogue, so their memory latency overlaps the O/LSE stores.
    WideItem cur, nxt;
    bool have = wide_item(p, 0, Gx, jw, x, Nx, BHx, ND, BM, BN, wave, cur);
    TL ld;
    WideRows<D> w;
    if (have) wide_item_issue<D, BN, NW>(p, cur, ld, lds, VOFF, TB, wave, lane, half, col, w.qf);

    for (int it = 0; have; ++it) {
        const int b = cur.b, hq = cur.hq;
        const int wrow0 = cur.wrow0;
        const int n_tiles = cur.n_tiles;
        const int NB = n_tiles * KB;

#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int qi = wrow0 + 32 * r + col;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) w.o[r][db] = f32x16_t{};
            w.s[r] = f32x16_t{};
            w.l_acc[r] = f32x4_t{};
            w.m_ref[r] = kNegInf;
            w.mc[r] = 0.0f;
            w.l_run[r] = 0.0f;
            w.lim[r] = p.causal ? qi + p.off : 0x7fffffff;
        }
        w.sel = rowsum_selector(lane);
        w.half = half;
        w.c = p.c;
        w.key_end = p.Sk;
        w.wmin_lim = p.causal ? wrow0 + p.off : 0x7fffffff;
        w.NBw = cur.NBw;

        // the item's copies and Q loads were issued before the previous
        // item's epilogue (or just above, for the first item)
        wait_vmem();
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            flip_q<D>(w.qf[r], p.qflip);
            // Q fragments are only ever MFMA B operands, which may sit in
            // AGPRs: put them there, out of the way of the VALU's registers
#pragma unroll
            for (int st = 0; st < QS; ++st) asm volatile("" : "+a"(w.qf[r][st]));
        }
        if (n_tiles > 0) {
            __syncthreads();
            if (w.NBw > 0) {
                // S(0), and the reference max from its exact (masked) row max
                wide_qk<D>(lds, off, w.qf, w.s);
                const bool m = w.needs_mask(0);
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    if (m) BlockOps<D>::mask(w.s[r], 0, half, w.key_end, w.lim[r]);
                    const float mx = BlockOps<D>::rowmax(w.s[r]);
                    w.m_ref[r] = mx;
                    w.mc[r] = (mx == kNegInf) ? 0.0f : mx * w.c;
                }
            }
        }
        // tile t lives in stage t % 3.  Tile 0 takes the general body; the
        // fast tiles [1, t_end) run with compile-time stage addresses, three
        // per trip from stage 1, then the one or two left (stages 1 and 2);
        // tile t_end may take the masked fast body; the tiles after it take
        // the general body (runtime stages).
        int t_end = 1;
        while (t_end < n_tiles && wide_fast_ok<KB>(t_end, w.NBw, w.key_end, w.wmin_lim)) ++t_end;
        int t = 0;
        if (n_tiles > 0) {
            wide_tile<D, BN, NW, false>(0, n_tiles, lds, lds + TB, lds + 2 * TB, ld, wave, lane,
                                        off, w);
            t = 1;
        }
        for (; t + 2 < t_end; t += 3) {
            wide_tile<D, BN, NW, true>(t, n_tiles, lds + TB, lds + 2 * TB, lds, ld, wave, lane,
                                       off, w);
            wide_tile<D, BN, NW, true>(t + 1, n_tiles, lds + 2 * TB, lds, lds + TB, ld, wave, lane,
                                       off, w);
            wide_tile<D, BN, NW, true>(t + 2, n_tiles, lds, lds + TB, lds + 2 * TB, ld, wave, lane,
                                       off, w);
        }
        // here t % 3 == 1: at most two fast tiles remain, in stages 1 and 2
        if (t < t_end) {
            wide_tile<D, BN, NW, true>(t, n_tiles, lds + TB, lds + 2 * TB, lds, ld, wave, lane,
                                       off, w);
            ++t;
        }
        if (t < t_end) {
            wide_tile<D, BN, NW, true>(t, n_tiles, lds + 2 * TB, lds, lds + TB, ld, wave, lane,
                                       off, w);
            ++t;
        }
        if (t < n_tiles && wide_masked_ok<KB>(t, w.NBw)) {
            const int sc = t % kPrefillStages;
            const int sn = sc == kPrefillStages - 1 ? 0 : sc + 1;
            const int sp = sc == 0 ? kPrefillStages - 1 : sc - 1;
            wide_tile<D, BN, NW, true, true>(t, n_tiles, lds + sc * TB, lds + sn * TB, lds + sp * TB,
                                             ld, wave, lane, off, w);
            ++t;
        }
        for (; t < n_tiles; ++t) {
            const int sc = t % kPrefillStages;
            const int sn = sc == kPrefillStages - 1 ? 0 : sc + 1;
            const int sp = sc == 0 ? kPrefillStages - 1 : sc - 1;
            wide_tile<D, BN, NW, false>(t, n_tiles, lds + sc * TB, lds + sn * TB, lds + sp * TB, ld,
                                        wave, lane, off, w);
        }
        // the last block's P V (its tile is still in place)
        if (NB > 0 && w.NBw == NB) {
            const char *Vl = lds + ((n_tiles - 1) % kPrefillStages) * TB + (KB - 1) * 32 * 2 * D;
#pragma unroll
            for (int ps = 0; ps < QS; ++ps) {
                const bf16x8_t a = wide_ld_v<D>(Vl, off, ps);
                const int t2 = ps / (D / 32), db = ps % (D / 32);
                w.o[0][db] = mfma32(a, w.pp[0][t2], w.o[0][db]);
                w.o[1][db] = mfma32(a, w.pp[1][t2], w.o[1][db]);
            }
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                w.l_acc[r] = mfma16(w.sel, w.pp[r][0], w.l_acc[r]);
                w.l_acc[r] = mfma16(w.sel, w.pp[r][1], w.l_acc[r]);
            }
        }
        __syncthreads();   // every wave is done with the LDS ring

        // the next item's first copies and Q loads, then this item's epilogue
        have = wide_item(p, it + 1, Gx, jw, x, Nx, BHx, ND, BM, BN, wave, nxt);
        if (have) wide_item_issue<D, BN, NW>(p, nxt, ld, lds, VOFF, TB, wave, lane, half, col, w.qf);

#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int qi = wrow0 + 32 * r + col;
            finish_rows<D, OUT_F32>(w.o[r], w.m_ref[r], w.l_run[r], w.l_acc[r][0], p.c, half, p.o,
                                    (((long)b * p.Sq + qi) * p.Hq + hq) * D,
                                    p.lse ? p.lse + ((long)b * p.Hq + hq) * p.Sq + qi : nullptr,
                                    qi < p.Sq);
        }
        cur = nxt;
    }
#endif
}

// ---------------------------------------------------------------------------
// Pipelined prefill for head dim 256: NW waves x 32 query rows of one (b, hq)
// per item, one wave per SIMD (Q and O alone take 192 registers per lane).
// 32-key blocks; step j issues the S^T MFMAs of block j + 1 and the P V
// MFMAs (and rounded-P row sums) of block j - 1, and computes P(j) on the
// VALU between them, so that no MFMA waits for the softmax.  Softmax: the
// lazy reference max of the 64-row kernel -- the exact row max of block 0,
// moved only when a block's exact P sum exceeds kWideOverflow in some lane
// (also inf / NaN), which then redoes that block against its exact max.
// K and V tiles (32 keys) have rings of their own, three stages each:
// block j's K is read in step j - 1 and its V in step j + 1.  Step j first
// waits for K(j + 1) and V(j - 1); its barrier then releases the stages of
// K(j) and V(j - 2), and the step copies K(j + 3) and V(j + 1) into them,
// each two steps before it is read.  Every wave issues 2 PER_WAVE copies per
// step; past the last block the copies read an empty range (zeros into a
// free stage), which keeps that count fixed.
// With 8 waves (head dim 128) the rings have six stages and the barrier
// comes before every second step only: the one before step 2m waits for
// K(2m + 1), K(2m + 2), V(2m - 1) and V(2m) and releases every stage read
// in steps up to 2m - 1; steps 2m and 2m + 1 copy K(j + 5) and V(j + 3)
// into stages read last in steps 2m - 2 and 2m - 1.
// ---------------------------------------------------------------------------
template <int D>
struct PipeRows {
    bf16x8_t qf[D / 16];   // Q fragment: B operand of the S^T MFMAs (AGPRs)
    f32x16_t o[D / 32];    // O^T
    f32x4_t l_acc;         // element 0: row sum of the rounded P (whole row)
    bf16x8_t sel;          // row-sum selector operand
    float m_ref;           // reference max (score units)
    float mc;              // c * m_ref, 0 while m_ref = -inf
    float l_run;           // exact row sum (this lane half)
    float c;
};

// Row block (32 rows) of wave `wave` within an item.  The waves of a
// workgroup are spread over the CU's four SIMDs in turn, so waves w and w + 4
// share one; in a causal item the diagonal work of a row block grows with
// its index, so with 8 waves the second four take the blocks in reverse
// order: SIMD s then holds blocks s and 7 - s, the same work on every SIMD.
// (The mapping only balances the SIMDs; any assignment is correct.)
template <int NW>
__device__ __forceinline__ int pipe_row_block(int wave)
{
    return (NW == 8 && wave >= 4) ? 11 - wave : wave;
}

// With two waves per SIMD (8 waves, VG) a lane has 256 registers, which the
// compiler splits evenly between VGPRs and AGPRs once a kernel uses any
// AGPR; 128 VGPRs spill S, P and the operands.  There every MFMA is inline
// asm with VGPR operands (the ping-pong kernel's forms, declared below): the
// P V and row-sum accumulators are read only by the later MFMAs of their
// chains or after pipe_drain_o, which the build's scan of the generated code
// checks.  The row sum's selector operand may be rematerialised right before
// its MFMA, so two wait states lead that one.
__device__ __forceinline__ void pp_mfma_first(f32x16_t &d, bf16x8_t a, bf16x8_t q);
__device__ __forceinline__ void pp_mfma_next(f32x16_t &d, bf16x8_t a, bf16x8_t q);
__device__ __forceinline__ void pp_mfma_pv(f32x16_t &o, bf16x8_t v, bf16x8_t p);
__device__ __forceinline__ void pipe_mfma_rowsum(f32x4_t &l, bf16x8_t sel, bf16x8_t p)
{
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0 ; accumulate-only"
                 : "+v"(l)
                 : "v"(sel), "v"(p));
}
// the wait for those MFMAs before the VALU reads O or the row sums (24 wait
// states; the 8-pass MFMA needs 13), with the accumulators as operands
template <int D>
__device__ __forceinline__ void pipe_drain_o(PipeRows<D> &w)
{
    static_assert(D / 32 == 4, "four O accumulators");
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+v"(w.o[0]), "+v"(w.o[1]), "+v"(w.o[2]), "+v"(w.o[3]), "+v"(w.l_acc)::"memory");
}

// Step j.  Kn: K rows of block j + 1 (S^T into sn); Vp: V rows of block
// j - 1 (P V with pp, its P; ACC = false: no such block); s: S^T(j),
// masked, turned into pw (P(j) as bf16 words) and la (its exact sum over
// this lane half) against the reference max.  Slot st issues S k-step st
// and P V step st with P(j)'s elements st * 16 / QS .. between them, and
// copy(st); the operand reads run kPipePF slots ahead.  kpre / vpre hold the
// operands of the step's first kPipePF slots on entry, and those of the next
// step (K rows at Kn2, V rows at Vn2) on return: before its last slot the
// step waits for its own reads, then takes the next step's barrier
// (sync_next; nothing where the next step has none) and reads them, so that
// the next step starts without waiting for LDS.
template <int D, bool VG, bool ACC, class CP, class SY>
__device__ __forceinline__ void pipe_step(PipeRows<D> &w, const OperandOffsets<D> &off,
                                          const char *Kn, const char *Vp, const f32x16_t &s,
                                          f32x16_t &sn, const bf16x8_t (&pp)[2],
                                          u32x4_t (&pw)[2], float &la, CP &&copy,
                                          const char *Kn2, const char *Vn2,
                                          bf16x8_t (&kpre)[kPipePF], bf16x8_t (&vpre)[kPipePF],
                                          SY &&sync_next)
{
    constexpr int QS = D / 16, DB = D / 32, EPS = 16 / QS;
    constexpr int PF = kPipePF;
    static_assert(PF < QS, "the prefetched slots are a prefix of the step");
    bf16x8_t ka[QS], va[QS];
    float y[16];
    auto rd = [&](int i) __attribute__((always_inline)) {
        ka[i] = wide_ld_k<D>(Kn, off, i);
        if (ACC) va[i] = wide_ld_v<D>(Vp, off, i);
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        ka[i] = kpre[i];
        va[i] = vpre[i];
    }
    la = -0.0f;   // -0 + x is x: the first add folds away
#pragma unroll
    for (int st = 0; st < QS; ++st) {
        const int t2 = st / DB, db = st % DB;
        if (st == QS - 1) {
            // every read of this step has been issued: wait for them, take
            // the next step's barrier and read its first operands
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            sync_next();
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                kpre[i] = wide_ld_k<D>(Kn2, off, i);
                vpre[i] = wide_ld_v<D>(Vn2, off, i);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (VG) {
            if (st == 0) pp_mfma_first(sn, ka[st], w.qf[st]);
            else pp_mfma_next(sn, ka[st], w.qf[st]);
        } else {
            if (st == 0) mfma_s_first(sn, ka[st], w.qf[st]);
            else mfma_s_next(sn, ka[st], w.qf[st]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (st + PF < QS) rd(st + PF);
#pragma unroll
        for (int i = 0; i < EPS; ++i) {
            const int r = st * EPS + i;
            y[r] = fast_exp2(fmaf(s[r], w.c, -w.mc));
            keep(y[r]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ACC) {
            if constexpr (VG) pp_mfma_pv(w.o[db], va[st], pp[t2]);
            else w.o[db] = mfma32(va[st], pp[t2], w.o[db]);
        }
        __builtin_amdgcn_sched_barrier(0);
        copy(st);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < EPS; ++i) {
            const int r = st * EPS + i;
            la += y[r];
            if (r & 1) {
                pw[r >> 3][(r >> 1) & 3] = pack_bf16(y[r - 1], y[r]);
                keep(pw[r >> 3][(r >> 1) & 3]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (ACC && st == QS - 1) {
            if constexpr (VG) {
                pipe_mfma_rowsum(w.l_acc, w.sel, pp[0]);
                pipe_mfma_rowsum(w.l_acc, w.sel, pp[1]);
            } else {
                w.l_acc = mfma16(w.sel, pp[0], w.l_acc);
                w.l_acc = mfma16(w.sel, pp[1], w.l_acc);
            }
        }
    }
    asm volatile("s_nop 7" : "+v"(sn)::"memory");
}

// After step j: where P(j) overflowed, redo it against the exact row max
// (s is block j's masked S^T); then add its exact sum.
template <int D, bool VG>
__device__ __forceinline__ void pipe_settle(PipeRows<D> &w, const f32x16_t &s, u32x4_t (&pw)[2],
                                            float &la)
{
    const bool big = !(la <= kWideOverflow);   // also true for inf and NaN
    if (__any(big)) {
        if constexpr (VG) pipe_drain_o(w);
        const float mx = BlockOps<D>::rowmax(s);
        const float m_new = fmaxf(w.m_ref, mx);
        const float alpha = (w.m_ref == kNegInf) ? 0.0f : fast_exp2((w.m_ref - m_new) * w.c);
        w.l_run *= alpha;
        w.l_acc[0] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int e = 0; e < 16; ++e) w.o[db][e] *= alpha;
            __builtin_amdgcn_sched_barrier(0);
        }
        w.m_ref = m_new;
        w.mc = (m_new == kNegInf) ? 0.0f : m_new * w.c;
        la = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) wide_pair<false>(s, q, w.c, w.mc, pw, la);
    }
    w.l_run += la;
}

template <int D, int NW, bool OUT_F32>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW == 8 ? 2 : 1)))
fa_prefill_pipe_kernel(const Params p)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    constexpr int BN = 32;
    constexpr int BM = 32 * NW;
    // two waves per SIMD (8 waves): all MFMAs inline asm with VGPR operands
    constexpr bool VG = NW == 8;
    constexpr int QS = D / 16;
    using TL = TileLoader<D, BN, NW>;
    using BO = BlockOps<D>;
    constexpr int TB = TL::TILE_BYTES;
    constexpr int BP = VG ? 2 : 1;         // steps per barrier
    constexpr int NSK = 3 * BP;            // K ring stages, then as many V stages
    constexpr int KA = NSK - BP + 1;       // step j copies K(j + KA) ...
    constexpr int VA = KA - 2;             // ... and V(j + VA)
    constexpr int VOFF = NSK * TB;         // V stage s sits at K stage s + VOFF
    constexpr int LPS = 2 * TL::PER_WAVE;  // copies per wave and step
    static_assert(BP * LPS <= 15, "vmcnt immediate");
    __shared__ __attribute__((aligned(1024))) char lds[2 * NSK * TB];
    static_assert(2 * NSK * TB <= 160 * 1024, "LDS");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;
    OperandOffsets<D> off;
    off.init(lane);
#pragma unroll
    for (int db = 0; db < OperandOffsets<D>::NV; ++db)
#pragma unroll
        for (int sec = 0; sec < 2; ++sec) {
            off.v[db][sec] += VOFF;
            // keep the bias inside the register: folded back into the
            // immediates it would overflow their 16 bits
            asm volatile("" : "+v"(off.v[db][sec]));
        }

    // byte offset of each of this lane's K / V row copies within a tile
    const int kstride = p.Hkv * D * 2;
    int loff[TL::PER_WAVE];
#pragma unroll
    for (int i = 0; i < TL::PER_WAVE; ++i) {
        const int row = (i * NW + wave) * TL::RPI + lane / TL::CPR;
        loff[i] = row * kstride + (((lane % TL::CPR) ^ swz<D>(row)) * 16);
    }
    // scale 0: S is 0 for every pair, which a zero Q gives exactly; with
    // c = 1 the mask's -inf then still gives P = 0
    const bool zero_scale = p.c == 0.0f;
    const float c = zero_scale ? 1.0f : p.c;

    const int BH = p.B * p.Hq;
    const int ND = p.domains;
    const int x = blockIdx.x % ND;
    const int jw = blockIdx.x / ND;
    const int Gx = gridDim.x / ND;
    const int BHx = BH / ND;
    const int Nx = BHx * p.n_mblocks;

    for (int it = 0; it * Gx < Nx; ++it) {
        const int li = it * Gx + ((it & 1) ? (Gx - 1 - jw) : jw);
        if (li >= Nx) continue;
        const int rank = p.head_major ? li % p.n_mblocks : li / BHx;
        const int bh = (p.head_major ? li / p.n_mblocks : li % BHx) * ND + x;
        const int mb = p.causal ? (p.n_mblocks - 1 - rank) : rank;
        const int b = bh / p.Hq;
        const int hq = bh % p.Hq;
        const int g = hq / p.group;
        const int row0 = mb * BM;
        const int wrow0 = row0 + pipe_row_block<NW>(wave) * 32;
        const int qi = wrow0 + col;
        const int last_row = min(row0 + BM, p.Sq) - 1;
        int NB = (p.Sk + BN - 1) / BN;   // blocks (= tiles) the workgroup walks
        if (p.causal) {
            const int hi = last_row + p.off;
            NB = hi < 0 ? 0 : min(NB, hi / BN + 1);
        }
        const int lim = p.causal ? qi + p.off : 0x7fffffff;
        const int wmin_lim = p.causal ? wrow0 + p.off : 0x7fffffff;
        auto needs_mask = [&](int j) __attribute__((always_inline)) { return j * 32 + 32 > p.Sk || j * 32 + 31 > wmin_lim; };

        const uint32_t kv_bytes = p.Sk > 0 ? (uint32_t)((p.Sk - 1) * kstride + D * 2) : 0u;
        const u32x4_t kd = raw_desc(p.k + ((long)b * p.Sk * p.Hkv + g) * D, kv_bytes);
        const u32x4_t vd = raw_desc(p.v + ((long)b * p.Sk * p.Hkv + g) * D, kv_bytes);
        // copy i of this wave's share of K(t) / V(t); past the last key the
        // byte range makes it zeros (offsets in unsigned arithmetic: the
        // tiles past the end may lie beyond 2 GiB)
        auto toff = [&](int t, int i) __attribute__((always_inline)) {
            return (int)((uint32_t)t * (uint32_t)(BN * kstride) + (uint32_t)loff[i]);
        };
        auto copy_k = [&](int t, int i) __attribute__((always_inline)) {
            lds_dma16(lds + (t % NSK) * TB + (i * NW + wave) * 1024, toff(t, i), kd);
        };
        auto copy_v = [&](int t, int i) __attribute__((always_inline)) {
            lds_dma16(lds + VOFF + (t % NSK) * TB + (i * NW + wave) * 1024, toff(t, i), vd);
        };

        PipeRows<D> w;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) w.o[db] = f32x16_t{};
        w.l_acc = f32x4_t{};
        w.sel = rowsum_selector(lane);
        w.m_ref = kNegInf;
        w.mc = 0.0f;
        w.l_run = 0.0f;
        w.c = c;

        if (NB > 0) {
#pragma unroll
            for (int i = 0; i < TL::PER_WAVE; ++i) copy_k(0, i);
        }
        load_q<D>(w.qf, p.q + (((long)b * p.Sq + min(qi, p.Sq - 1)) * p.Hq + hq) * D, half);
        wait_vmem();
        if (zero_scale) {
#pragma unroll
            for (int st = 0; st < QS; ++st) w.qf[st] = bf16x8_t{};
        }
        flip_q<D>(w.qf, p.qflip);
        // Q fragments are only ever B operands of inline-asm MFMAs: AGPRs
        // (one wave per SIMD), VGPRs (two)
#pragma unroll
        for (int st = 0; st < QS; ++st) {
            if constexpr (VG) asm volatile("" : "+v"(w.qf[st]));
            else asm volatile("" : "+a"(w.qf[st]));
        }
        __syncthreads();   // K(0) is in LDS (every wave's copies)

        if (NB > 0) {
            // the copies steps 1 - KA .. -1 would have issued: K(t + KA) and
            // V(t + VA) for each of them, V of a block before 0 being
            // nothing (an empty range into its free stage)
            const u32x4_t none = raw_desc(p.v, 0u);
#pragma unroll
            for (int t = 1 - KA; t < 0; ++t) {
#pragma unroll
                for (int i = 0; i < TL::PER_WAVE; ++i) copy_k(t + KA, i);
#pragma unroll
                for (int i = 0; i < TL::PER_WAVE; ++i) {
                    if (t + VA >= 0)
                        copy_v(t + VA, i);
                    else
                        lds_dma16(lds + VOFF + ((t + VA + NSK) % NSK) * TB + (i * NW + wave) * 1024,
                                  loff[i], none);
                }
            }

            f32x16_t sx, sy;                 // S^T of the even / odd block
            bf16x8_t px[2], py[2];           // P of the even / odd block
            u32x4_t pw[2];
            float la;
            // S(0) and the reference max from its exact (masked) row max
            {
                bf16x8_t ka[QS];
#pragma unroll
                for (int st = 0; st < QS; ++st) ka[st] = wide_ld_k<D>(lds, off, st);
#pragma unroll
                for (int st = 0; st < QS; ++st) {
                    if constexpr (VG) {
                        if (st == 0) pp_mfma_first(sx, ka[st], w.qf[st]);
                        else pp_mfma_next(sx, ka[st], w.qf[st]);
                    } else {
                        if (st == 0) mfma_s_first(sx, ka[st], w.qf[st]);
                        else mfma_s_next(sx, ka[st], w.qf[st]);
                    }
                }
                mfma_s_drain(sx);
                if (needs_mask(0)) BO::mask(sx, 0, half, p.Sk, lim);
                const float mx = BO::rowmax(sx);
                w.m_ref = mx;
                w.mc = (mx == kNegInf) ? 0.0f : mx * c;
            }
            // the wave's last key block with an allowed key (-1: none).  Its
            // later blocks are masked out entirely, so the steps past them
            // are skipped: with two waves per SIMD that gives the SIMD to the
            // other wave, whose rows reach further
            int Lw = NB - 1;
            {
                const int wlast = min(wrow0 + 31, p.Sq - 1);
                if (wlast < wrow0)
                    Lw = -1;
                else if (p.causal)
                    Lw = wlast + p.off < 0 ? -1 : min(NB - 1, (wlast + p.off) / 32);
            }
            // the barrier before step j (every BP-th step): wait for K(j + 1)
            // and V(j - 1) (with BP = 2 also K(j + 2) and V(j); the copies of
            // the BP steps before may stay in flight), then every wave's.
            // Step j copies K(j + KA) and V(j + VA) in its first slots.  Step
            // j - 1 takes the barrier before its last slot, once all its
            // reads (of the stages the next BP steps refill) are in
            static_assert(LPS <= D / 16 - 1, "a step's copies go out before its last slot");
            auto sync = [&]() __attribute__((always_inline)) {
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(0x0F70 | (BP * LPS));
                pp_barrier();
            };
            auto no_sync = [&]() __attribute__((always_inline)) {};
            auto copies = [&](int j) __attribute__((always_inline)) {
                return [&, j](int st) __attribute__((always_inline)) {
                    if (st < TL::PER_WAVE) copy_k(j + KA, st);
                    else if (st < 2 * TL::PER_WAVE) copy_v(j + VA, st - TL::PER_WAVE);
                };
            };
            // the operands of each step's first slots, read at the end of the
            // step before (step 0's here: K(1); it has no P V)
            bf16x8_t kpre[kPipePF], vpre[kPipePF];
            sync();
#pragma unroll
            for (int i = 0; i < kPipePF; ++i) {
                kpre[i] = wide_ld_k<D>(lds + TB, off, i);
                vpre[i] = bf16x8_t{};
            }
            // each step before a barrier takes it before its last slot
            if constexpr (BP == 1)
                pipe_step<D, VG, false>(w, off, lds + TB, lds, sx, sy, py, pw, la, copies(0),
                                        lds + 2 * TB, lds, kpre, vpre, sync);
            else
                pipe_step<D, VG, false>(w, off, lds + TB, lds, sx, sy, py, pw, la, copies(0),
                                        lds + 2 * TB, lds, kpre, vpre, no_sync);
            pipe_settle<D, VG>(w, sx, pw, la);
            px[0] = __builtin_bit_cast(bf16x8_t, pw[0]);
            px[1] = __builtin_bit_cast(bf16x8_t, pw[1]);
            // step j >= 1: the register sets of block j (even: sx / px, odd:
            // sy / py) follow from its parity, and its ring stage j % NSK is
            // a compile-time constant (STAGE), so that every LDS address of
            // the step is a lane offset plus an immediate
            auto step = [&](auto odd, auto stage, int j) __attribute__((always_inline)) {
                constexpr bool ODD = decltype(odd)::value;
                constexpr int ST = decltype(stage)::value;
                const char *Kn = lds + ((ST + 1) % NSK) * TB;
                const char *Vp = lds + ((ST + NSK - 1) % NSK) * TB;   // + VOFF in the offsets
                f32x16_t &s = ODD ? sy : sx;
                f32x16_t &sn = ODD ? sx : sy;
                bf16x8_t(&pp)[2] = ODD ? px : py;
                bf16x8_t(&pn)[2] = ODD ? py : px;
                if (needs_mask(j)) BO::mask(s, j * 32, half, p.Sk, lim);
                // the next step reads K(j + 2) and V(j); with BP = 2 only the
                // odd steps take a barrier (the one before the even step)
                if constexpr (BP == 1 || ODD)
                    pipe_step<D, VG, true>(w, off, Kn, Vp, s, sn, pp, pw, la, copies(j),
                                           lds + ((ST + 2) % NSK) * TB, lds + ST * TB, kpre,
                                           vpre, sync);
                else
                    pipe_step<D, VG, true>(w, off, Kn, Vp, s, sn, pp, pw, la, copies(j),
                                           lds + ((ST + 2) % NSK) * TB, lds + ST * TB, kpre,
                                           vpre, no_sync);
                pipe_settle<D, VG>(w, s, pw, la);
                pn[0] = __builtin_bit_cast(bf16x8_t, pw[0]);
                pn[1] = __builtin_bit_cast(bf16x8_t, pw[1]);
            };
            using T = std::true_type;
            using F = std::false_type;
            // the steps this wave computes: its live blocks, and the P V of
            // the last (later steps only take the ring's barriers and copies)
            const int NBw = min(NB, Lw + 2);
            int j = 1;
            // six steps per trip (j = 1 mod 6), then the rest
            using S1 = std::integral_constant<int, 1 % NSK>;
            using S2 = std::integral_constant<int, 2 % NSK>;
            using S3 = std::integral_constant<int, 3 % NSK>;
            using S4 = std::integral_constant<int, 4 % NSK>;
            using S5 = std::integral_constant<int, 5 % NSK>;
            using S6 = std::integral_constant<int, 6 % NSK>;
            for (; j + 5 < NBw; j += 6) {
                step(T{}, S1{}, j);
                step(F{}, S2{}, j + 1);
                step(T{}, S3{}, j + 2);
                step(F{}, S4{}, j + 3);
                step(T{}, S5{}, j + 4);
                step(F{}, S6{}, j + 5);
            }
            // the rest: at most five steps, from j = 1 mod 6
            if (j < NBw) step(T{}, S1{}, j);
            if (j + 1 < NBw) step(F{}, S2{}, j + 1);
            if (j + 2 < NBw) step(T{}, S3{}, j + 2);
            if (j + 3 < NBw) step(F{}, S4{}, j + 3);
            if (j + 4 < NBw) step(T{}, S5{}, j + 4);
            // dead steps: their copies, and the barriers the other waves take
            // (the one before step jd + 1 where BP divides jd + 1)
            for (int jd = max(1, NBw); jd < NB; ++jd) {
                auto cp = copies(jd);
#pragma unroll
                for (int st = 0; st < LPS; ++st) cp(st);
                if (BP == 1 || ((jd + 1) & 1) == 0) sync();
            }
            // the last block's P V: V(NB - 1) is in (the last step took the
            // barrier after it; that step's own copies may stay in flight)
            if (NB - 1 <= Lw) {
            bf16x8_t pl[2];
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                pl[t2] = (NB & 1) ? px[t2] : py[t2];
                // the select is a VALU write of an MFMA operand: two wait states
                if constexpr (VG) asm volatile("s_nop 1" : "+v"(pl[t2]));
            }
            const char *Vl = lds + ((NB - 1) % NSK) * TB;
#pragma unroll
            for (int ps = 0; ps < QS; ++ps) {
                const int t2 = ps / (D / 32), db = ps % (D / 32);
                if constexpr (VG) pp_mfma_pv(w.o[db], wide_ld_v<D>(Vl, off, ps), pl[t2]);
                else w.o[db] = mfma32(wide_ld_v<D>(Vl, off, ps), pl[t2], w.o[db]);
            }
            if constexpr (VG) {
                pipe_mfma_rowsum(w.l_acc, w.sel, pl[0]);
                pipe_mfma_rowsum(w.l_acc, w.sel, pl[1]);
            } else {
                w.l_acc = mfma16(w.sel, pl[0], w.l_acc);
                w.l_acc = mfma16(w.sel, pl[1], w.l_acc);
            }
            }
        }
        if constexpr (VG) pipe_drain_o(w);
        __syncthreads();   // every wave is done with the rings before the next item

        finish_rows<D, OUT_F32>(w.o, w.m_ref, w.l_run, w.l_acc[0], c, half, p.o,
                                (((long)b * p.Sq + qi) * p.Hq + hq) * D,
                                p.lse ? p.lse + ((long)b * p.Hq + hq) * p.Sq + qi : nullptr,
                                qi < p.Sq);
    }
#endif
}

// ---------------------------------------------------------------------------
// Pipelined FP8 prefill (D = 128): 8 waves x 32 query rows = 256 rows of one
// (b, hq) per item, two waves per SIMD.  The operands are those of
// fa_prefill_fp8_kernel: E4M3 tiles with rows of D bytes, the 32x32x64 FP8
// MFMA, P rounded to E4M3, V^T through the 8-bit transposing read.  The steps
// are those of fa_prefill_pipe_kernel, on blocks of 64 keys (one FP8 MFMA per
// 32 head dims of P V): step j issues the four S^T MFMAs of block j + 1 and
// the four P V MFMAs of block j - 1 (then its rounded-P row sum) and computes
// P(j) on the VALU between them, a quarter per MFMA pair, so that neither
// unit waits for the other's results.
// Softmax: the lazy reference max -- the exact row max of block 0, moved only
// when a block's exact P sum passes kFp8PipeOverflow = 2^8 in some lane (also
// inf / NaN), which redoes that block against its exact row max.  Each P is
// then below 2^8, inside E4M3's largest value 448.
// K and V have three-stage rings of their own (8 KiB per stage): step j waits
// for K(j + 1) and V(j - 1), and after its barrier copies K(j + 3) and
// V(j + 1) into the stages of K(j) and V(j - 2) from inside its first slots;
// past the last block the copies read an empty range, which keeps the count
// of copies per step fixed for vmcnt.
// Registers: two waves per SIMD leave 256 per lane, which the compiler splits
// evenly between VGPRs and AGPRs as soon as a kernel uses AGPRs at all, and
// 128 VGPRs do not hold S, P and the operands.  So every MFMA here is inline
// asm with VGPR operands and accumulators, and the kernel uses no AGPR.  The
// S^T accumulators are fenced at the end of each step (the VALU reads them in
// the next one); O and the row sums are read only by the later MFMAs of their
// chains, which the hardware orders, or after fp8_drain_o.  The build's scan
// of the generated code checks the wait states around each of them.
// ---------------------------------------------------------------------------
constexpr float kFp8PipeOverflow = 256.0f;
constexpr int kFp8PipeWaves = 8;

// The FP8 MFMA (16 passes): S^T with a VGPR accumulator ...
__device__ __forceinline__ void mfma_s8_first(f32x16_t &d, i32x8_t a, i32x8_t b)
{
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s8_next(f32x16_t &d, i32x8_t a, i32x8_t b)
{
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// ... O^T += V^T P^T ("accumulate-only": the build's scan follows a branch
// past it instead of reporting it) ...
__device__ __forceinline__ void mfma_o8(f32x16_t &o, i32x8_t a, i32x8_t b)
{
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0 ; accumulate-only"
                 : "+v"(o)
                 : "v"(a), "v"(b));
}
// ... and the row sums of the rounded P against the all-ones A operand,
// which the compiler may rematerialise right before it: two wait states lead
// (a VALU write of an MFMA source needs two).
__device__ __forceinline__ void mfma_rowsum8(f32x16_t &l, i32x8_t ones, i32x8_t p)
{
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0 ; accumulate-only"
                 : "+v"(l)
                 : "v"(ones), "v"(p));
}

__device__ __forceinline__ i32x8_t fp8_ones()
{
    constexpr int kOnes = 0x38383838;   // E4M3 1.0 in every byte
    return (i32x8_t){kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes};
}

template <int D>
struct Fp8PipeRows {
    i32x8_t qf[D / 64];   // Q fragments: B operands of the S^T MFMAs
    f32x16_t o[D / 32];   // O^T
    f32x16_t l_acc;       // element 0: row sum of the rounded P (whole row)
    float m_ref;          // reference max (score units)
    float mc;             // c * m_ref, 0 while m_ref = -inf
    float l_run;          // exact row sum (this lane half)
    float c;
    i32x8_t ones;         // E4M3 1.0 in every byte: A operand of the row sums
};

// The wait for the P V and row-sum MFMAs before the VALU reads O or the row
// sums: 24 wait states (the 16-pass MFMA needs 21), with the accumulators as
// operands, so that nothing the compiler emits can touch them before it.
template <int D>
__device__ __forceinline__ void fp8_drain_o(Fp8PipeRows<D> &w)
{
    static_assert(D / 32 == 4, "four O accumulators");
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+v"(w.o[0]), "+v"(w.o[1]), "+v"(w.o[2]), "+v"(w.o[3]), "+v"(w.l_acc)::"memory");
}

// A operand of S^T MFMA m of a 64-key block (K rows at Kblk): key half
// m / KS, k-step m % KS.
template <int D>
__device__ __forceinline__ i32x8_t fp8_ld_k(const char *Kblk, const Fp8Offsets<D> &off, int m)
{
    constexpr int KS = D / 64;
    const int kb = m / KS, st = m % KS;
    const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(Kblk + kb * 32 * D + off.k[st][0]);
    const u32x4_t hi = *reinterpret_cast<const u32x4_t *>(Kblk + kb * 32 * D + off.k[st][1]);
    return (i32x8_t){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// A operand V^T of P V MFMA db (head dims 32 db .. 32 db + 31, the block's
// 64 keys in the byte order of P): four 8-bit transposing reads.
template <int D>
__device__ __forceinline__ i32x8_t fp8_ld_v(const char *Vblk, const Fp8Offsets<D> &off, int db)
{
    i32x8_t a;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
        const i32x2_t w =
            __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t *)(Vblk + off.vofs(db, t4)));
        a[2 * t4] = w[0];
        a[2 * t4 + 1] = w[1];
    }
    return a;
}

// y[0..3] as E4M3 bytes (round to nearest even), byte order of the P V
// MFMA's B operand.  Both halves of the word are written, so the register
// the first conversion merges into needs no value: an empty asm statement
// hands one over, which spares the compiler a move that zeroes or copies it.
__device__ __forceinline__ int fp8_word(const float *y)
{
    int old;
    asm volatile("" : "=v"(old));
    const int word = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], old, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], word, true);
}

// Step j.  Kn: K rows of block j + 1 (S^T into sn); Vp: V rows of block
// j - 1 (P V with pp, its P; ACC = false: no such block); s: S^T(j), masked,
// turned into pw (P(j) as E4M3 bytes, byte 16 kb + r of the B operand) and la
// (its exact sum over this lane half) against the reference max.  Slot m
// issues S MFMA m and P V MFMA m with P(j)'s elements 8m .. 8m + 7 between
// them, and copy(m); each slot's operands are read one slot ahead.  kpre
// holds the first slot's K operand on entry, and the next step's (K rows at
// Kn2) on return: before its last slot the step waits for its own reads,
// takes the next step's barrier (sync_next) and reads it.  (The V operand of
// a step's first slot is read at its start: its P V MFMA comes second.)
template <int D, bool ACC, class CP, class SY>
__device__ __forceinline__ void fp8_pipe_step(Fp8PipeRows<D> &w, const Fp8Offsets<D> &off,
                                              const char *Kn, const char *Vp,
                                              const f32x16_t (&s)[2], f32x16_t (&sn)[2],
                                              const i32x8_t &pp, i32x8_t &pw, float &la, CP &&copy,
                                              const char *Kn2, i32x8_t &kpre, SY &&sync_next)
{
    constexpr int KS = D / 64, DB = D / 32, NM = 2 * KS;
    static_assert(NM == DB, "one S^T and one P V MFMA per slot");
    i32x8_t ka[NM], va[DB];
    float y[32];
    auto rd = [&](int i) __attribute__((always_inline)) {
        ka[i] = fp8_ld_k<D>(Kn, off, i);
        if (ACC) va[i] = fp8_ld_v<D>(Vp, off, i);
    };
    ka[0] = kpre;
    if (ACC) va[0] = fp8_ld_v<D>(Vp, off, 0);
    la = -0.0f;   // -0 + x is x: the first add folds away
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int kb = m / KS, st = m % KS;
        if (m == NM - 1) {
            // every read of this step has been issued: wait for them, take
            // the next step's barrier and read its first operands
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            sync_next();
            kpre = fp8_ld_k<D>(Kn2, off, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (st == 0) mfma_s8_first(sn[kb], ka[m], w.qf[st]);
        else mfma_s8_next(sn[kb], ka[m], w.qf[st]);
        __builtin_amdgcn_sched_barrier(0);
        if (m + 1 < NM) rd(m + 1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = 8 * m + i;
            y[e] = fast_exp2(fmaf(s[e >> 4][e & 15], w.c, -w.mc));
            keep(y[e]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (ACC) mfma_o8(w.o[m], va[m], pp);
        __builtin_amdgcn_sched_barrier(0);
        copy(m);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int e = 8 * m + 4 * h;
            pw[2 * m + h] = fp8_word(&y[e]);
            keep((uint32_t)pw[2 * m + h]);
            la += (y[e] + y[e + 1]) + (y[e + 2] + y[e + 3]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (ACC) mfma_rowsum8(w.l_acc, w.ones, pp);
    asm volatile("s_nop 7" : "+v"(sn[0]), "+v"(sn[1])::"memory");
}

// After step j: where P(j) overflowed, redo it against the exact row max
// (s is block j's masked S^T); then add its exact sum.
template <int D>
__device__ __forceinline__ void fp8_pipe_settle(Fp8PipeRows<D> &w, const f32x16_t (&s)[2],
                                                i32x8_t &pw, float &la)
{
    const bool big = !(la <= kFp8PipeOverflow);   // also true for inf and NaN
    if (__any(big)) {
        fp8_drain_o(w);
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
        mx = max_halves(mx);
        const float m_new = fmaxf(w.m_ref, mx);
        const float alpha = (w.m_ref == kNegInf) ? 0.0f : fast_exp2((w.m_ref - m_new) * w.c);
        w.l_run *= alpha;
        w.l_acc[0] *= alpha;   // only element 0 of the row-sum accumulator is read
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int e = 0; e < 16; ++e) w.o[db][e] *= alpha;
            __builtin_amdgcn_sched_barrier(0);
        }
        w.m_ref = m_new;
        w.mc = (m_new == kNegInf) ? 0.0f : m_new * w.c;
        float y[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) y[e] = fast_exp2(fmaf(s[e >> 4][e & 15], w.c, -w.mc));
        la = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            pw[q] = fp8_word(&y[4 * q]);
            la += (y[4 * q] + y[4 * q + 1]) + (y[4 * q + 2] + y[4 * q + 3]);
        }
    }
    w.l_run += la;
}

template <int D, bool OUT_F32>
__global__ void __launch_bounds__(kFp8PipeWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
fa_prefill_fp8_pipe_kernel(const Params p, const float v_descale)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    static_assert(D == 128, "the FP8 operand offsets assume head dim 128");
    constexpr int NW = kFp8PipeWaves;
    constexpr int BN = 64;
    constexpr int BM = 32 * NW;
    constexpr int KS = D / 64;
    constexpr int RB = D;                   // bytes per tile row
    constexpr int CPR = RB / 16;            // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;           // rows per copy instruction
    constexpr int PER_WAVE = BN / RPI / NW; // copies per wave, tensor and tile
    static_assert(PER_WAVE >= 1 && PER_WAVE * RPI * NW == BN, "copies split evenly");
    constexpr int TB = BN * RB;             // 8 KiB per tile
    constexpr int NSK = 3;                  // K ring stages, then as many V stages
    constexpr int VOFF = NSK * TB;          // V stage s sits at K stage s + VOFF
    constexpr int LPS = 2 * PER_WAVE;       // copies per wave and step
    static_assert(LPS <= 2 * KS, "the copies go out in the step's first slots");
    __shared__ __attribute__((aligned(1024))) char lds[2 * NSK * TB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;
    Fp8Offsets<D> off;
    off.init(lane);
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) off.vb[t4] += VOFF;

    const uint8_t *q8 = reinterpret_cast<const uint8_t *>(p.q);
    const uint8_t *k8 = reinterpret_cast<const uint8_t *>(p.k);
    const uint8_t *v8 = reinterpret_cast<const uint8_t *>(p.v);

    // byte offset of each of this lane's K / V row copies within a tile
    const int kstride = p.Hkv * D;
    int loff[PER_WAVE];
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int row = (i * NW + wave) * RPI + lane / CPR;
        loff[i] = row * kstride + (((lane % CPR) ^ swz_fp8(row)) * 16);
    }
    // scale 0: S is 0 for every pair, which a zero Q gives exactly; with
    // c = 1 the mask's -inf then still gives P = 0
    const bool zero_scale = p.c == 0.0f;
    const float c = zero_scale ? 1.0f : p.c;

    const int BH = p.B * p.Hq;
    const int ND = p.domains;
    const int x = blockIdx.x % ND;
    const int jw = blockIdx.x / ND;
    const int Gx = gridDim.x / ND;
    const int BHx = BH / ND;
    const int Nx = BHx * p.n_mblocks;

    for (int it = 0; it * Gx < Nx; ++it) {
        const int li = it * Gx + ((it & 1) ? (Gx - 1 - jw) : jw);
        if (li >= Nx) continue;
        const int rank = p.head_major ? li % p.n_mblocks : li / BHx;
        const int bh = (p.head_major ? li / p.n_mblocks : li % BHx) * ND + x;
        const int mb = p.causal ? (p.n_mblocks - 1 - rank) : rank;
        const int b = bh / p.Hq;
        const int hq = bh % p.Hq;
        const int g = hq / p.group;
        const int row0 = mb * BM;
        const int wrow0 = row0 + pipe_row_block<NW>(wave) * 32;
        const int qi = wrow0 + col;
        const int last_row = min(row0 + BM, p.Sq) - 1;
        int NB = (p.Sk + BN - 1) / BN;   // blocks (= tiles) the workgroup walks
        if (p.causal) {
            const int hi = last_row + p.off;
            NB = hi < 0 ? 0 : min(NB, hi / BN + 1);
        }
        const int lim = p.causal ? qi + p.off : 0x7fffffff;
        const int wmin_lim = p.causal ? wrow0 + p.off : 0x7fffffff;
        auto needs_mask = [&](int j) __attribute__((always_inline)) {
            return j * BN + BN > p.Sk || j * BN + BN - 1 > wmin_lim;
        };
        auto mask = [&](f32x16_t (&s)[2], int j) __attribute__((always_inline)) {
            BlockOps<64>::mask(s[0], j * BN, half, p.Sk, lim);
            BlockOps<64>::mask(s[1], j * BN + 32, half, p.Sk, lim);
        };

        const uint32_t kv_bytes = p.Sk > 0 ? (uint32_t)((p.Sk - 1) * kstride + D) : 0u;
        const u32x4_t kd = raw_desc(k8 + ((long)b * p.Sk * p.Hkv + g) * D, kv_bytes);
        const u32x4_t vd = raw_desc(v8 + ((long)b * p.Sk * p.Hkv + g) * D, kv_bytes);
        // copy i of this wave's share of K(t) / V(t); past the last key the
        // byte range makes it zeros (offsets in unsigned arithmetic: the
        // tiles past the end may lie beyond 2 GiB)
        auto toff = [&](int t, int i) __attribute__((always_inline)) {
            return (int)((uint32_t)t * (uint32_t)(BN * kstride) + (uint32_t)loff[i]);
        };
        auto copy_k = [&](int t, int i) __attribute__((always_inline)) {
            lds_dma16(lds + (t % NSK) * TB + (i * NW + wave) * 1024, toff(t, i), kd);
        };
        auto copy_v = [&](int t, int i) __attribute__((always_inline)) {
            lds_dma16(lds + VOFF + (t % NSK) * TB + (i * NW + wave) * 1024, toff(t, i), vd);
        };

        Fp8PipeRows<D> w;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) w.o[db] = f32x16_t{};
        w.l_acc = f32x16_t{};
        w.m_ref = kNegInf;
        w.mc = 0.0f;
        w.l_run = 0.0f;
        w.c = c;
        w.ones = fp8_ones();

        if (NB > 0) {
#pragma unroll
            for (int i = 0; i < PER_WAVE; ++i) copy_k(0, i);
        }
        {
            // this lane's Q bytes: k-step st, dims 64 st + 32 half .. + 31
            const uint8_t *qrow = q8 + (((long)b * p.Sq + min(qi, p.Sq - 1)) * p.Hq + hq) * D;
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                const u32x4_t lo =
                    ld16(reinterpret_cast<const uint16_t *>(qrow + 64 * st + 32 * half));
                const u32x4_t hi =
                    ld16(reinterpret_cast<const uint16_t *>(qrow + 64 * st + 32 * half + 16));
                w.qf[st] = (i32x8_t){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
        }
        wait_vmem();
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            if (zero_scale) w.qf[st] = i32x8_t{};
            // a negative scale negates Q exactly (E4M3 sign bits)
            if (p.qflip) w.qf[st] ^= (int)0x80808080u;
            asm volatile("" : "+v"(w.qf[st]));
        }
        __syncthreads();   // K(0) is in LDS (every wave's copies)

        if (NB > 0) {
            // the copies steps -2 and -1 would have issued: K(1) and V(-1)
            // (nothing: an empty range into V(2)'s stage), then K(2) and V(0)
            const u32x4_t none = raw_desc(v8, 0u);
#pragma unroll
            for (int i = 0; i < PER_WAVE; ++i) copy_k(1, i);
#pragma unroll
            for (int i = 0; i < PER_WAVE; ++i)
                lds_dma16(lds + VOFF + 2 * TB + (i * NW + wave) * 1024, loff[i], none);
#pragma unroll
            for (int i = 0; i < PER_WAVE; ++i) copy_k(2, i);
#pragma unroll
            for (int i = 0; i < PER_WAVE; ++i) copy_v(0, i);

            f32x16_t sx[2], sy[2];   // S^T of the even / odd block
            i32x8_t px, py;          // P of the even / odd block
            i32x8_t pw;
            float la;
            // S(0) and the reference max from its exact (masked) row max
            {
                i32x8_t ka[2 * KS];
#pragma unroll
                for (int m = 0; m < 2 * KS; ++m) ka[m] = fp8_ld_k<D>(lds, off, m);
#pragma unroll
                for (int m = 0; m < 2 * KS; ++m) {
                    const int kb = m / KS, st = m % KS;
                    if (st == 0) mfma_s8_first(sx[kb], ka[m], w.qf[st]);
                    else mfma_s8_next(sx[kb], ka[m], w.qf[st]);
                }
                mfma_s_drain(sx[0], sx[1]);
                if (needs_mask(0)) mask(sx, 0);
                float mx = kNegInf;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sx[kb][e]);
                mx = max_halves(mx);
                w.m_ref = mx;
                w.mc = (mx == kNegInf) ? 0.0f : mx * c;
            }
            // the barrier before step j: wait for K(j + 1) and V(j - 1) (the
            // copies of step j - 1 may stay in flight), then every wave's;
            // step j copies K(j + 3) and V(j + 1) in its first slots.  Step
            // j - 1 takes it before its last slot, once all its reads (of
            // K(j) and V(j - 2), whose stages step j refills) are in
            static_assert(LPS <= 2 * KS - 1, "a step's copies go out before its last slot");
            auto sync = [&]() __attribute__((always_inline)) {
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(0x0F70 | LPS);
                pp_barrier();
            };
            // the wave's last key block with an allowed key (-1: none).  Its
            // later blocks are masked out entirely, so the steps past them
            // are skipped: that gives the SIMD to the other wave on it
            int Lw = NB - 1;
            {
                const int wlast = min(wrow0 + 31, p.Sq - 1);
                if (wlast < wrow0)
                    Lw = -1;
                else if (p.causal)
                    Lw = wlast + p.off < 0 ? -1 : min(NB - 1, (wlast + p.off) / BN);
            }
            auto copies = [&](int j) __attribute__((always_inline)) {
                return [&, j](int m) __attribute__((always_inline)) {
                    if (m < PER_WAVE) copy_k(j + 3, m);
                    else if (m < 2 * PER_WAVE) copy_v(j + 1, m - PER_WAVE);
                };
            };
            // the K operand of each step's first slot, read at the end of the
            // step before (step 0's here: K(1))
            sync();
            i32x8_t kpre = fp8_ld_k<D>(lds + TB, off, 0);
            // each step takes the next one's barrier before its last slot
            fp8_pipe_step<D, false>(w, off, lds + TB, lds, sx, sy, py, pw, la, copies(0),
                                    lds + 2 * TB, kpre, sync);
            fp8_pipe_settle<D>(w, sx, pw, la);
            px = pw;
            // step j >= 1: the register sets of block j (even: sx / px, odd:
            // sy / py) follow from its parity, and its ring stage j % 3 is a
            // compile-time constant, so that every LDS address of the step
            // is a lane offset plus an immediate
            auto step = [&](auto odd, auto stage, int j) __attribute__((always_inline)) {
                constexpr bool ODD = decltype(odd)::value;
                constexpr int ST = decltype(stage)::value;
                const char *Kn = lds + ((ST + 1) % NSK) * TB;
                const char *Vp = lds + ((ST + NSK - 1) % NSK) * TB;   // + VOFF in the offsets
                f32x16_t(&s)[2] = ODD ? sy : sx;
                f32x16_t(&sn)[2] = ODD ? sx : sy;
                i32x8_t &pp = ODD ? px : py;
                i32x8_t &pn = ODD ? py : px;
                if (needs_mask(j)) mask(s, j);
                // the next step reads K(j + 2) first
                fp8_pipe_step<D, true>(w, off, Kn, Vp, s, sn, pp, pw, la, copies(j),
                                       lds + ((ST + 2) % NSK) * TB, kpre, sync);
                fp8_pipe_settle<D>(w, s, pw, la);
                pn = pw;
            };
            using T = std::true_type;
            using F = std::false_type;
            // the steps this wave computes: its live blocks, and the P V of
            // the last (later steps only take the ring's barriers and copies)
            const int NBw = min(NB, Lw + 2);
            int j = 1;
            // six steps per trip (j = 1 mod 6), then the rest
            for (; j + 5 < NBw; j += 6) {
                step(T{}, std::integral_constant<int, 1>{}, j);
                step(F{}, std::integral_constant<int, 2>{}, j + 1);
                step(T{}, std::integral_constant<int, 0>{}, j + 2);
                step(F{}, std::integral_constant<int, 1>{}, j + 3);
                step(T{}, std::integral_constant<int, 2>{}, j + 4);
                step(F{}, std::integral_constant<int, 0>{}, j + 5);
            }
            // the rest: at most five steps, from j = 1 mod 6
            if (j < NBw) step(T{}, std::integral_constant<int, 1>{}, j);
            if (j + 1 < NBw) step(F{}, std::integral_constant<int, 2>{}, j + 1);
            if (j + 2 < NBw) step(T{}, std::integral_constant<int, 0>{}, j + 2);
            if (j + 3 < NBw) step(F{}, std::integral_constant<int, 1>{}, j + 3);
            if (j + 4 < NBw) step(T{}, std::integral_constant<int, 2>{}, j + 4);
            for (int jd = max(1, NBw); jd < NB; ++jd) {
                auto cp = copies(jd);
#pragma unroll
                for (int m = 0; m < LPS; ++m) cp(m);
                sync();
            }
            // the last block's P V: V(NB - 1) is in (the last step took the
            // barrier after it; that step's own copies may stay in flight)
            if (NB - 1 <= Lw) {
                i32x8_t pl = (NB & 1) ? px : py;
                // the select is a VALU write of an MFMA operand: two wait states
                asm volatile("s_nop 1" : "+v"(pl));
                const char *Vl = lds + ((NB - 1) % NSK) * TB;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    mfma_o8(w.o[db], fp8_ld_v<D>(Vl, off, db), pl);
                mfma_rowsum8(w.l_acc, w.ones, pl);
            }
        }
        fp8_drain_o(w);
        __syncthreads();   // every wave is done with the rings before the next item

        // O = v_descale * O / l: the descale folds into the normaliser
        finish_rows<D, OUT_F32>(w.o, w.m_ref, w.l_run, w.l_acc[0] / v_descale, c, half, p.o,
                                (((long)b * p.Sq + qi) * p.Hq + hq) * D,
                                p.lse ? p.lse + ((long)b * p.Hq + hq) * p.Sq + qi : nullptr,
                                qi < p.Sq);
    }
#endif
}

// ---------------------------------------------------------------------------
// Ping-pong prefill: 8 waves x 32 query rows = 256 rows of one (b, hq) per
// item, two waves per SIMD.  Waves 0-3 (group A) and 4-7 (group B) share the
// SIMDs pairwise and run the same two-phase loop half a period apart:
//
//   M(t): S(t) = K(t) Q^T (2 key blocks x D/16 MFMAs) and O += V(t-1)^T P(t-1)^T
//         (4 x D/32 MFMAs), plus the row sums of the rounded P(t-1);
//   V(t): the online softmax that turns S(t) into P(t) (VALU only).
//
//   phase:   0     1     2     3     4   ...   2T   2T+1
//   group A  M(0)  V(0)  M(1)  V(1)  M(2)      M(T)  -
//   group B  -     M(0)  V(0)  M(1)  V(1)      V(T-1) M(T)
//
// A workgroup barrier closes every phase, so on each SIMD one wave issues
// MFMAs while the other runs its softmax: measured on gfx950, an MFMA-only
// wave keeps its 32-cycle issue rate beside a VALU-only wave, whereas one
// wave interleaving both loses about 12 cycles of VALU issue per MFMA.  This
// is the SIMD-level form of the overlap the FlashAttention page describes for
// SM90 (softmax of one tile under the matrix work of another, "SM80 内核实现对比",
// section 5.2), without its warp specialisation: every wave does both kinds
// of work, in alternation.
//
// K/V: 64-key tiles in an NS-stage LDS ring (K tiles, then V tiles).  Tile t
// is read in M(t) (K) and M(t+1) (V), i.e. in phases 2t .. 2t+3, so its stage
// is free from phase 2t+4 on.  Every wave copies its share of each tile at
// the start of one of its V phases, into a stage that is already free then:
// group A (V(t) in phase 2t+1) tile t + NS - 2, into the stage of tile t - 2;
// group B (V(t) in phase 2t+2) tile t + NS - 1, into the stage of tile t - 1.
// Tile t + 1 is read from phase 2t+2 on, so both groups wait for their copies
// of it in phase 2t+1 (A at the end of V(t), B at the end of M(t)), before the
// barrier; the copies have 2 NS - 6 (A) and 2 NS - 5 (B) phases to land.
//
// Softmax: V(0) (and any tile that is masked or partly dead for the wave)
// uses the exact running max; the other tiles use the lazy reference max of
// the wide kernel above: P = exp2(c s - c m_ref) without a max, redone against
// the exact max when a lane's P sum exceeds kWideOverflow (also inf / NaN).
// ---------------------------------------------------------------------------
constexpr int kPPWaves = 8;
constexpr int kPPBN = 64;

template <int D>
struct PPRows {
    static constexpr int QS = D / 16, DB = D / 32;
    bf16x8_t qf[QS];
    f32x16_t o[DB];
    f32x16_t s[2];         // S^T of the current tile, key blocks 0 and 1
    bf16x8_t p[4];         // P of the previous tile, 16-key steps 0..3
    f32x4_t l_acc;         // element 0: row sum of the rounded P (whole row)
    float m_ref, l_run;    // reference max (score units), exact row sum (lane half)
    bf16x8_t sel;
};

// LDS reads at a 32-bit LDS byte address (the constant part of the address
// folds into the instruction's offset field).
__device__ __forceinline__ bf16x8_t lds_read16(uint32_t addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t *>((uintptr_t)addr);
}
// A operand V^T of a 16-key P V step: two transposing reads (keys k0 + 4 h
// + 0..3 and k0 + 8 + 4 h + 0..3 of 4 head dims), from the lane addresses of
// OperandOffsets::v.
__device__ __forceinline__ bf16x8_t lds_read_vt(uint32_t a0, uint32_t a1)
{
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<lds_i16x4_t *>((uintptr_t)a0));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<lds_i16x4_t *>((uintptr_t)a1));
    const u32x2_t lw = __builtin_bit_cast(u32x2_t, lo);
    const u32x2_t hw = __builtin_bit_cast(u32x2_t, hi);
    return __builtin_bit_cast(bf16x8_t, (u32x4_t){lw[0], lw[1], hw[0], hw[1]});
}

// Per-lane LDS addresses of one phase's operand reads: the tile's base plus
// the lane's offsets, formed once per phase behind an opaque value, so that
// the compiler does not keep a register for every (stage, step) combination.
template <int D>
struct PPAddr {
    uint32_t k[D / 16];      // K fragment of k-step st (key block 0; block 1 is +32 rows)
    uint32_t v[D / 32][2];   // V^T halves of d block db (16-key step 0; step t2 is +16 t2 rows)
    __device__ __forceinline__ void set(uint32_t kbase, uint32_t vbase, const OperandOffsets<D> &off)
    {
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            k[st] = kbase + (uint32_t)off.kofs(st);
            asm volatile("" : "+v"(k[st]));
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int sec = 0; sec < 2; ++sec) {
                v[db][sec] = vbase + (uint32_t)off.vofs(db, sec);
                asm volatile("" : "+v"(v[db][sec]));
            }
    }
};

// The M phase's MFMAs as inline asm with tied accumulators, so that O, S and
// the row sums keep their registers through the phase (with the builtins the
// register allocator moved O between register sets, copying it every phase).
// The compiler's hazard recognizer does not see inside, so:
//  * S is complete before the V phase reads it: the S MFMAs are issued in
//    the first part of the M phase, and about half the phase's P V MFMAs
//    follow the last of them;
//  * pp_drain_o precedes every VALU access to O and the row sums (the
//    rescale after an overflow, the epilogue);
//  * an M phase starts with two wait states (s_nop 1) after the VALU writes
//    of P and O of the phase before it;
//  * operand registers are rewritten by the rolling reads at least three
//    steps after the MFMA that read them.
__device__ __forceinline__ void pp_mfma_first(f32x16_t &d, bf16x8_t a, bf16x8_t q)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(q));
}
__device__ __forceinline__ void pp_mfma_next(f32x16_t &d, bf16x8_t a, bf16x8_t q)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(q));
}
// O and the row sums are read only by the next MFMAs of their chains or after
// pp_drain_o / the fenced wait of the rescale path: the build's device-code
// scan lets a branch follow these MFMAs closely (the "accumulate-only" mark)
// and checks the fall-through code instead.
__device__ __forceinline__ void pp_mfma_pv(f32x16_t &o, bf16x8_t v, bf16x8_t p)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0 ; accumulate-only"
                 : "+v"(o)
                 : "v"(v), "v"(p));
}
__device__ __forceinline__ void pp_mfma_rowsum(f32x4_t &l, bf16x8_t sel, bf16x8_t p)
{
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0 ; accumulate-only"
                 : "+v"(l)
                 : "v"(sel), "v"(p));
}

// Wait for the P V and row-sum MFMAs before the VALU reads O or the row
// sums (24 wait states; an 8-pass MFMA needs about half): the accumulators
// are operands, so nothing the compiler emits can touch them before it.
template <int D>
__device__ __forceinline__ void pp_drain_o(PPRows<D> &w)
{
    if constexpr (D / 32 == 4)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+v"(w.o[0]), "+v"(w.o[1]), "+v"(w.o[2]), "+v"(w.o[3]),
                       "+v"(w.l_acc)::"memory");
    else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+v"(w.o[0]), "+v"(w.o[1]), "+v"(w.l_acc)::"memory");
}

// The same wait for S, after an M phase that ends with S MFMAs.
template <int D>
__device__ __forceinline__ void pp_drain_s(PPRows<D> &w)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(w.s[0]), "+v"(w.s[1])::"memory");
}

// M phase.  DO_S: S(t) of both key blocks of tile t; DO_PV: O += V^T P^T for
// both blocks of tile t - 1, and the row sums of the rounded P; operand
// addresses from `ad` (formed during the V phase before).  Blocks dead for
// this wave are computed too (their K and V rows are in range) and get P = 0
// in the V phase: no conditional writes, so the compiler keeps S and P in
// place.  Operand reads run two steps ahead of their MFMAs.  The S MFMAs go
// first, two per P V MFMA, so that S is complete long before the V phase
// reads it (the last S MFMA is followed by about half the P V MFMAs); O and
// the row sums are waited for only where the VALU reads them (pp_drain_o).
template <int D, bool DO_S, bool DO_PV>
__device__ __forceinline__ void pp_mphase(const PPAddr<D> &ad, PPRows<D> &w)
{
    constexpr int QS = D / 16, DB = D / 32;
    constexpr int NSM = DO_S ? 2 * QS : 0;    // S MFMAs
    constexpr int NPV = DO_PV ? 4 * DB : 0;   // P V MFMAs (4 steps of 16 keys x DB)
    // step order: S steps at twice the rate of P V steps while both remain
    constexpr int N = NSM + NPV;
    auto is_s = [&](int j) {   // step j is an S step, and which one
        if (!DO_PV) return true;
        if (!DO_S) return false;
        return j < 3 * (NSM / 2) ? (j % 3) != 2 : false;
    };
    auto idx = [&](int j) {    // index of step j among its kind
        if (!DO_PV) return j;
        if (!DO_S) return j;
        if (j < 3 * (NSM / 2)) return (j % 3) != 2 ? 2 * (j / 3) + (j % 3) : j / 3;
        return j - NSM;
    };
    auto ldk = [&](int i) {   // S step i: kb = i % 2, st = i / 2
        return lds_read16(ad.k[i >> 1] + (i & 1) * 32 * 2 * D);
    };
    auto ldv = [&](int i) {   // P V step i: t2 = i / DB, db = i % DB
        const int t2 = i / DB, db = i % DB;
        return lds_read_vt(ad.v[db][0] + t2 * 16 * 2 * D, ad.v[db][1] + t2 * 16 * 2 * D);
    };
    set_prio<1>();
    asm volatile("s_nop 1" ::: "memory");
    bf16x8_t op[3];   // operand reads two steps ahead (rolling)
#pragma unroll
    for (int j = 0; j < 2 && j < N; ++j) op[j] = is_s(j) ? ldk(idx(j)) : ldv(idx(j));
#pragma unroll
    for (int j = 0; j < N; ++j) {
        if (j + 2 < N) op[(j + 2) % 3] = is_s(j + 2) ? ldk(idx(j + 2)) : ldv(idx(j + 2));
        const int i = idx(j);
        if (is_s(j)) {
            const int kb = i & 1, st = i >> 1;
            if (st == 0)
                pp_mfma_first(w.s[kb], op[j % 3], w.qf[st]);
            else
                pp_mfma_next(w.s[kb], op[j % 3], w.qf[st]);
        } else {
            const int t2 = i / DB, db = i % DB;
            pp_mfma_pv(w.o[db], op[j % 3], w.p[t2]);
            if (db == DB - 1) pp_mfma_rowsum(w.l_acc, w.sel, w.p[t2]);
        }
    }
    set_prio<0>();
}

// P of one key block from its S (16 registers) against c * m_ref = mc,
// packed to bf16 as the B operands of two 16-key P V steps; la adds the
// exact values.  MASK: keys past `last` (offset from this lane half's first
// key of the block) get exponent -inf, i.e. P = 0 for any scale.
template <bool MASK>
__device__ __forceinline__ void pp_probs(const f32x16_t &s, float c, float mc, int last,
                                         bf16x8_t &p0, bf16x8_t &p1, float &la)
{
    u32x4_t w0, w1;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        float x0 = fmaf(s[2 * q], c, -mc);
        float x1 = fmaf(s[2 * q + 1], c, -mc);
        if (MASK) {
            const int e0 = 2 * q, e1 = 2 * q + 1;
            x0 = (8 * (e0 >> 2) + (e0 & 3) > last) ? kNegInf : x0;
            x1 = (8 * (e1 >> 2) + (e1 & 3) > last) ? kNegInf : x1;
        }
        const float a = fast_exp2(x0), b = fast_exp2(x1);
        if (q < 4)
            w0[q] = pack_bf16(a, b);
        else
            w1[q - 4] = pack_bf16(a, b);
        la += a + b;
    }
    p0 = __builtin_bit_cast(bf16x8_t, w0);
    p1 = __builtin_bit_cast(bf16x8_t, w1);
}

// V phase with the exact running max: blocks at or past `live` are dead
// (P = 0), keys past the lane's limit are masked.  key0: the tile's first
// key.  Returns the factor the caller applies to O and the row sums.
template <int D>
__device__ __forceinline__ float pp_vphase_exact(PPRows<D> &w, int live, int key0, int half,
                                                 int lim, float c)
{
    int last[2];
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        // largest allowed key offset from this lane half's first key of the block
        last[kb] = kb < live ? lim - (key0 + kb * 32 + 4 * half) : -1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const bool ok = 8 * (r >> 2) + (r & 3) <= last[kb];
            mx = fmaxf(mx, ok ? w.s[kb][r] : kNegInf);
        }
    }
    mx = max_halves(mx);
    const float m_new = fmaxf(w.m_ref, mx);
    // nothing accumulated yet (m_ref = -inf): O and the sums are zero
    float alpha = 1.0f;
    if (w.m_ref == kNegInf)
        alpha = 0.0f;
    else if (m_new > w.m_ref)
        alpha = fast_exp2((w.m_ref - m_new) * c);
    w.m_ref = m_new;
    const float mc = (m_new == kNegInf) ? 0.0f : m_new * c;
    float la = 0.0f;
    pp_probs<true>(w.s[0], c, mc, last[0], w.p[0], w.p[1], la);
    pp_probs<true>(w.s[1], c, mc, last[1], w.p[2], w.p[3], la);
    w.l_run = w.l_run * alpha + la;
    return alpha;
}

// V phase: P(t) from S(t).  Tiles whose two blocks are live and unmasked for
// the wave, after the reference max is set (FAST), skip the max and redo the
// tile against the exact max only when a lane's P sum overflows; O and the
// rounded-P row sum are rescaled on that path only.
template <int D>
__device__ __forceinline__ void pp_vphase(PPRows<D> &w, bool fast, int live, int key0, int half,
                                          int lim, float c)
{
    constexpr int DB = D / 32;
    bool redo = !fast;
    if (fast) {
        const float mc = w.m_ref * c;
        float la = -0.0f;
        pp_probs<false>(w.s[0], c, mc, 0, w.p[0], w.p[1], la);
        pp_probs<false>(w.s[1], c, mc, 0, w.p[2], w.p[3], la);
        // !(x <= T) is also true for inf and NaN
        redo = __any(!(la <= kWideOverflow));
        if (!redo) w.l_run += la;
    }
    float alpha = 1.0f;
    if (redo) {
        // the wait for the last P V and row-sum MFMAs before O and the row
        // sums are read; fenced rather than tied to O (tying O to an asm
        // statement in this branch costs the copies described below)
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        alpha = pp_vphase_exact<D>(w, live, key0, half, lim, c);
    }
    // written after the branch on purpose: the compiler folds it away on the
    // common path (alpha = 1 there), whereas a rescale written inside the
    // branch made the register allocator keep two homes for O and copy it
    // every phase
    w.l_acc[0] *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) w.o[db][e] *= alpha;
}

template <int D, int NS, bool OUT_F32>
__global__ void __launch_bounds__(kPPWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
fa_prefill_pp_kernel(const Params p)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    constexpr int NW = kPPWaves, BN = kPPBN, BM = 32 * NW;
    using TL = TileLoader<D, BN, NW>;
    constexpr int TB = TL::TILE_BYTES;
    constexpr int VOFF = NS * TB;   // V tile s sits at K tile s + VOFF
    constexpr int CPW = 2 * TL::PER_WAVE;   // copy instructions per wave and tile
    static_assert(NS >= 4 && NS <= 5, "ring depth");

    __shared__ __attribute__((aligned(1024))) char lds[2 * NS * TB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;          // 0: group A, 1: group B
    const int col = lane & 31;
    const int half = lane >> 5;

    OperandOffsets<D> off;
    off.init(lane);
#pragma unroll
    for (int db = 0; db < OperandOffsets<D>::NV; ++db)
#pragma unroll
        for (int sec = 0; sec < 2; ++sec) off.v[db][sec] += VOFF;
    const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>((lds_void_t *)lds);

    const int BH = p.B * p.Hq;
    const int ND = p.domains;
    const int x = blockIdx.x % ND;
    const int jw = blockIdx.x / ND;
    const int Gx = gridDim.x / ND;
    const int BHx = BH / ND;
    const int Nx = BHx * p.n_mblocks;

    // item `it` of this workgroup: (b, hq, query block), snake order
    auto item = [&](int it, int &b, int &hq, int &row0, int &T) {
        if (it * Gx >= Nx) return false;
        const int li = it * Gx + ((it & 1) ? (Gx - 1 - jw) : jw);
        if (li >= Nx) return false;
        const int rank = p.head_major ? li % p.n_mblocks : li / BHx;
        const int bh = (p.head_major ? li / p.n_mblocks : li % BHx) * ND + x;
        const int mb = p.causal ? (p.n_mblocks - 1 - rank) : rank;
        b = bh / p.Hq;
        hq = bh % p.Hq;
        row0 = mb * BM;
        const int last_row = min(row0 + BM, p.Sq) - 1;
        int n = (p.Sk + BN - 1) / BN;
        if (p.causal) {
            const int hi = last_row + p.off;
            n = hi < 0 ? 0 : min(n, hi / BN + 1);
        }
        T = n;
        return true;
    };
    // each of the 8 waves copies an eighth of every tile
    TL ld;
    auto issue_item = [&](int b, int hq, int row0, int T, PPRows<D> &w) {
        const int g = hq / p.group;
        ld.setup(p.k + ((long)b * p.Sk * p.Hkv + g) * D, p.v + ((long)b * p.Sk * p.Hkv + g) * D,
                 p.Hkv * D * 2, p.Sk);
        if (T > 0) ld.issue(lds, lds + VOFF, 0, wave, lane);
        const int qi = min(row0 + 32 * wave + col, p.Sq - 1);
        load_q<D>(w.qf, p.q + (((long)b * p.Sq + qi) * p.Hq + hq) * D, half);
#pragma unroll
        for (int u = 1; u < NS; ++u)
            if (u < T) ld.issue(lds + u * TB, lds + VOFF + u * TB, u * BN, wave, lane);
    };

    PPRows<D> w;
    int b = 0, hq = 0, row0 = 0, T = 0;
    bool have = item(0, b, hq, row0, T);
    if (have) issue_item(b, hq, row0, T, w);

    for (int it = 0; have; ++it) {
        const int wrow0 = row0 + 32 * wave;
        const int qi = wrow0 + col;
        const int wlast = min(wrow0 + 31, p.Sq - 1);
        // key blocks this wave has work on (a prefix), and the smallest and
        // this lane's causal limits
        int NBw;
        if (wrow0 >= p.Sq)
            NBw = 0;
        else if (p.causal) {
            const int wmax_lim = wlast + p.off;
            NBw = wmax_lim < 0 ? 0 : min(2 * T, wmax_lim / 32 + 1);
        } else
            NBw = 2 * T;
        const int wmin_lim = p.causal ? wrow0 + p.off : 0x7fffffff;
        const int lim = min(p.causal ? qi + p.off : 0x7fffffff, p.Sk - 1);
        const int key_end = p.Sk;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) w.o[db] = f32x16_t{};
        w.l_acc = f32x4_t{};
        w.m_ref = kNegInf;
        w.l_run = 0.0f;
        w.sel = rowsum_selector(lane);

        // Q and tile 0 landed; later tiles may be in flight
        wait_tiles_ahead<CPW, 4>(min(NS - 1, T - 1));
        flip_q<D>(w.qf, p.qflip);
        pp_barrier();

        // a tile's blocks: live count for this wave, and whether any key of
        // a live block is cut by the causal limit or the key end
        auto live_of = [&](int t) { return max(0, min(2, NBw - 2 * t)); };
        auto clean = [&](int t) {
            return (2 * t + 1) * 32 + 31 <= wmin_lim && (2 * t + 2) * 32 <= key_end;
        };
        auto kbase = [&](int k) { return lds_base + (k % NS) * TB; };
        // every V phase writes all of P (0 for dead blocks and masked keys)
        auto vphase = [&](int k) {
            const int live = live_of(k);
            pp_vphase<D>(w, k >= 1 && live == 2 && clean(k), live, k * BN, half, lim, p.c);
        };
        // operand addresses of M(k): K tile k, V tile k - 1
        PPAddr<D> ad;
        auto addr = [&](int k) { ad.set(kbase(k), kbase(k + NS - 1), off); };
        // tile k + 1 is read from phase 2k+2 on: this wave's copies of it
        // have landed (later tiles may still be in flight) ...
        auto wait_next = [&](int k) {
            if (k + 1 < T) {
                const int issued_last = min(T - 1, max(NS - 1, k + NS - 2));
                wait_tiles_ahead<CPW, 4>(issued_last - (k + 1));
            }
        };
        // ... and every wave's after the barrier that follows.  This wave's
        // share of the next tile its V(k) may fill (see above).
        auto refill = [&](int k) {
            const int u = k + NS - 2 + grp;
            if (u >= NS && u < T)
                ld.issue(lds + (u % NS) * TB, lds + VOFF + (u % NS) * TB, u * BN, wave, lane);
        };
        // Both groups run the same sequence M(0) V(0) M(1) V(1) ... M(T),
        // one barrier after every phase; group B starts one barrier late and
        // group A ends one barrier late, so that their phases alternate.
        if (T > 0) {
            addr(0);
            if (grp == 1) pp_barrier();
            pp_mphase<D, true, false>(ad, w);
            pp_drain_s<D>(w);
            if (grp == 1) wait_next(0);
            pp_barrier();
            vphase(0);
            addr(1);
            if (grp == 0) wait_next(0);
            pp_barrier();
            for (int k = 1; k < T; ++k) {
                pp_mphase<D, true, true>(ad, w);
                if (grp == 1) wait_next(k);
                pp_barrier();
                refill(k);
                vphase(k);
                addr(k + 1);
                if (grp == 0) wait_next(k);
                pp_barrier();
            }
            pp_mphase<D, false, true>(ad, w);
            pp_barrier();
            if (grp == 0) pp_barrier();
        }
        pp_drain_o<D>(w);

        // this item's stores, then (the ring is free) the next item's copies
        // and Q: the item start waits for the stores, Q and the first tile
        // only, since vector-memory operations complete in issue order
        finish_rows<D, OUT_F32>(w.o, w.m_ref, w.l_run, w.l_acc[0], p.c, half, p.o,
                                (((long)b * p.Sq + qi) * p.Hq + hq) * D,
                                p.lse ? p.lse + ((long)b * p.Hq + hq) * p.Sq + qi : nullptr,
                                qi < p.Sq);
        int nb = 0, nhq = 0, nrow0 = 0, nT = 0;
        have = item(it + 1, nb, nhq, nrow0, nT);
        if (have) issue_item(nb, nhq, nrow0, nT, w);
        b = nb;
        hq = nhq;
        row0 = nrow0;
        T = nT;
    }
#endif
}

// ---------------------------------------------------------------------------
// Split-key decode: one wave per (b, KV head g, split).  Its 32 MFMA columns
// are the (query row, head-in-group) pairs of KV head g: column j is query
// j / group, head g * group + j % group; columns >= Sq * group are padding.
// ---------------------------------------------------------------------------
template <int D, bool OUT_F32>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(D >= 256 ? 1 : 2)))
fa_decode_split_kernel(const Params p)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    constexpr int BN = kDecodeBN;
    using WT = WaveTile<D, BN>;
    using TL = TileLoader<D, BN, 1, true>;
    constexpr int TB = TL::TILE_BYTES;
    constexpr int STAGE = 2 * TB;

    constexpr int S = kDecodeStages;
    // D >= 256: K tile n in K stage n % KS, V tile n in V stage n % VS
    constexpr int KS = kDecodeKStages256, VS = kDecodeVStages256;
    constexpr int LDS_BYTES = D >= 256 ? (KS + VS) * TB : S * STAGE;
    __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];

    const int lane = threadIdx.x;
    const int col = lane & 31;
    const int half = lane >> 5;

    OperandOffsets<D> off;
    off.init(lane);

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
    const int k_end = min(k_begin + p.split_len, p.Sk);
    const int n_tiles = k_end > k_begin ? (k_end - k_begin + BN - 1) / BN : 0;

    bf16x8_t qf[D / 16];

    TL ld;
    ld.setup(p.k + ((long)b * p.Sk * p.Hkv + g) * D, p.v + ((long)b * p.Sk * p.Hkv + g) * D,
             p.Hkv * D * 2, k_end);

    f32x16_t o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
    float m_ref = kNegInf, l_run = 0.0f, l_rnd = 0.0f;

    const int lim_lane = p.causal ? qi + p.off : 0x7fffffff;
    const int wmin_lim = p.causal ? p.off : 0x7fffffff;   // row 0 has the smallest limit

    // the first tiles' copies go out together, then Q (padding columns load
    // a real row: they are never written).  D >= 256: K(0), V(0), K(1);
    // otherwise the first S - 1 tiles.
    char *const kring = lds, *const vring = lds + KS * TB;
    if constexpr (D >= 256) {
        if (n_tiles > 0) {
            ld.template issue_one<false>(kring, k_begin, 0, lane);
            ld.template issue_one<true>(vring, k_begin, 0, lane);
        }
        if (n_tiles > 1) ld.template issue_one<false>(kring + TB, k_begin + BN, 0, lane);
    } else {
#pragma unroll
        for (int u = 0; u < S - 1; ++u)
            if (u < n_tiles)
                ld.issue(lds + u * STAGE, lds + u * STAGE + TB, k_begin + u * BN, 0, lane);
    }
    load_q<D>(qf, p.q + (((long)b * p.Sq + qi) * p.Hq + hq) * D, half);
    flip_q<D>(qf, p.qflip);
    // Q has landed, and with it every copy issued before it.  Saying so
    // explicitly clears the compiler's record of loads in flight; without it
    // the compiler kept one path's Q loads pending and put a vmcnt(0) at the
    // top of the key loop, draining the ring once per trip.
    wait_vmem();
    if constexpr (D >= 256) {
        // one tile per trip, stage offsets at run time (an unrolled trip does
        // not fit the register file at D = 256).  A 32-key tile is 16 copies
        // per tensor, so vmcnt (at most 63) could cover only one whole tile
        // ahead with a common ring; with separate rings the copies in flight
        // are V(n + 1), K(n + 1) and K(n + 2), 48 KiB, in 80 KiB of LDS:
        // two workgroups per CU.  Copies go out in the order V(n), K(n + 1),
        // so tile n has landed once at most K(n + 1)'s 16 are outstanding.
        constexpr int LPT = TL::PER_WAVE;
        int ks = 0, vs = 0;
        for (int n = 0; n < n_tiles; ++n) {
            if (n + 1 < n_tiles)
                __builtin_amdgcn_s_waitcnt((LPT & 15) | ((LPT >> 4) << 14) | 0x0F70);
            else
                wait_vmem();
            // one wave: orders its LDS reads of tile n - 1 before the copies
            // below overwrite its stages
            __syncthreads();
            if (n + 1 < n_tiles)
                ld.template issue_one<true>(vring + (vs ^ 1) * TB, k_begin + (n + 1) * BN, 0,
                                            lane);
            if (n + 2 < n_tiles) {
                const int k2 = ks + 2 >= KS ? ks + 2 - KS : ks + 2;
                ld.template issue_one<false>(kring + k2 * TB, k_begin + (n + 2) * BN, 0, lane);
            }
            const int key0 = k_begin + n * BN;
            WaveTile<D, BN>::template step<true>(kring + ks * TB, vring + vs * TB, off, qf, o,
                                                 m_ref, l_run, l_rnd, p.c, half, key0, k_end,
                                                 lim_lane);
            ks = ks + 1 == KS ? 0 : ks + 1;
            vs ^= 1;
        }
    } else {
        // S tiles per trip keep every stage offset a compile-time constant
        for (int n = 0; n < n_tiles; n += S) {
#pragma unroll
            for (int u = 0; u < S; ++u)
                if (n + u < n_tiles)
                    decode_step<D, BN, S, TL>(n + u, n_tiles, k_begin, lds, u, ld, lane, k_end,
                                              wmin_lim, off, qf, o, m_ref, l_run, l_rnd, p.c,
                                              half, lim_lane);
        }
    }

    const float l_norm = add_halves(l_rnd);
    if (p.num_splits == 1) {
        finish_rows<D, OUT_F32>(o, m_ref, l_run, l_norm, p.c, half, p.o,
                                (((long)b * p.Sq + qi) * p.Hq + hq) * D,
                                p.lse ? p.lse + ((long)b * p.Hq + hq) * p.Sq + qi : nullptr, valid);
    } else {
        const long prow = (((long)s * p.B + b) * p.Hq + hq) * p.Sq + qi;
        finish_rows<D, true>(o, m_ref, l_run, l_norm, p.c, half, p.part_o, prow * D,
                             p.part_lse + prow, valid);
    }
#endif
}

// ---------------------------------------------------------------------------
// Split-key decode over a paged K/V cache (PagedTileLoader): as
// fa_decode_split_kernel, except that sequence b has its own length
// seq_lens[b] (clamped to [0, max_pages * page_size]) and its own causal
// offset, and its keys are cut into num_splits equal ranges, multiples of the
// tile, so that every split of a sequence streams about the same bytes.
// Splits past the end of a short sequence write an empty partial (O_s = 0,
// LSE_s = -inf), which the merge weighs 0.
// ---------------------------------------------------------------------------
struct PagedParams {
    const int *table;        // [B][max_pages]
    const int *seq_lens;     // [B]
    int max_pages, num_pages, lg_page;
    // length-balanced ranges (balanced != 0): see paged_range_tiles
    int balanced;
    int slots;               // resident (range, KV head) waves the CUs hold at once
    int range_cap;           // ranges the grid and the workspace provide for
    int len_min, len_max;    // bounds of the common range length (multiples of kDecodeBN)
    int *range_info;         // [B][2]: each sequence's first range and range count
};

// ---- length-balanced key ranges of the paged decode ---------------------------
// Every sequence's keys are cut into ranges of one common length L: the
// shortest multiple of the tile in [len_min, len_max] for which the (range,
// KV head) items fit the CUs' resident slots in one round.  A long sequence
// then gets more ranges than a short one, no item streams more than L keys,
// and no slot waits for a second round (waves and tail: "理解 H100：从硬件数据
// 路径到 Nsight Compute 瓶颈分析", section 2).  When even len_max needs more
// items than slots, L = len_max.  The lengths live on the device, so every
// wave derives L (a binary search over the range count, which falls as L
// grows), and the range its item stands for, from seq_lens itself: no
// planning pass and no host synchronisation.  Ranges are numbered sequence by
// sequence: sequence b owns ranges [first_b, first_b + n_b), n_b = ceil(Sk_b /
// L).  The host sizes range_cap >= max(slots / Hkv, B ceil(capacity /
// len_max)), which the count never exceeds.
__device__ __forceinline__ int paged_seq_len(const PagedParams &pp, int b)
{
    return min(max(pp.seq_lens[b], 0), pp.max_pages << pp.lg_page);
}

// Wave-wide integer sum and inclusive prefix sum on DPP moves within rows of
// 16 lanes and four v_readlane of the row totals: a few dozen cycles, where
// the same through the LDS crossbar (ds_bpermute) costs a round trip per step.
// The sum comes back as a scalar (uniform).
#define FA_DPP(x, ctrl) __builtin_amdgcn_update_dpp(0, (x), (ctrl), 0xf, 0xf, true)

__device__ __forceinline__ int wave_sum_i32(int x)
{
    x += FA_DPP(x, 0xB1);    // quad_perm [1,0,3,2]
    x += FA_DPP(x, 0x4E);    // quad_perm [2,3,0,1]: every lane holds its quad's sum
    x += FA_DPP(x, 0x124);   // row_ror:4
    x += FA_DPP(x, 0x128);   // row_ror:8: every lane holds its row's sum
    return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) +
           __builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48);
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane)
{
    x += FA_DPP(x, 0x111);   // row_shr:1 (lanes shifted in from outside the row read 0)
    x += FA_DPP(x, 0x112);   // row_shr:2
    x += FA_DPP(x, 0x114);   // row_shr:4
    x += FA_DPP(x, 0x118);   // row_shr:8: inclusive prefix within each row of 16
    const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
              r2 = __builtin_amdgcn_readlane(x, 47);
    const int row = lane >> 4;
    return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}
#undef FA_DPP

// The tiles (kDecodeBN keys) of sequences 64 r + lane, r < 4, 0 past B: the
// balanced cut serves at most kPagedBalancedMaxSeqs = 256 sequences, whose
// lengths each wave then keeps in four registers (one memory round trip,
// however many times the search below counts ranges).
static_assert(kPagedBalancedMaxSeqs == 4 * 64, "four registers of 64 lanes");
struct PagedTiles {
    int t[4];
    int nreg;   // registers in use: ceil(B / 64), uniform
};

__device__ __forceinline__ PagedTiles paged_tiles(const PagedParams &pp, int B, int lane)
{
    PagedTiles pt;
    pt.nreg = (B + 63) / 64;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        // a clamped load and a select: no divergent region
        const int b = 64 * r + lane;
        const int v = r < pt.nreg ? paged_seq_len(pp, min(b, B - 1)) : 0;
        pt.t[r] = b < B ? (v + kDecodeBN - 1) / kDecodeBN : 0;
    }
    return pt;
}

// Sequence b's tiles (b uniform), as a scalar.
__device__ __forceinline__ int paged_tiles_of(const PagedTiles &pt, int b)
{
    const int r = b >> 6;
    const int v = r == 0 ? pt.t[0] : r == 1 ? pt.t[1] : r == 2 ? pt.t[2] : pt.t[3];
    return __builtin_amdgcn_readlane(v, b & 63);
}

// The number of ranges of lt tiles each (all 64 lanes of the wave call this).
__device__ __forceinline__ int paged_range_count(const PagedTiles &pt, int lt)
{
    int n = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (r < pt.nreg) n += (pt.t[r] + lt - 1) / lt;   // a uniform branch
    return wave_sum_i32(n);
}

// The common range length, in tiles (all 64 lanes of the wave call this).
__device__ __forceinline__ int paged_range_tiles(const PagedParams &pp, const PagedTiles &pt,
                                                 int Hkv)
{
    const int target = max(1, pp.slots / Hkv);
    int lo = pp.len_min / kDecodeBN, hi = pp.len_max / kDecodeBN;
    if (paged_range_count(pt, hi) > target) return hi;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (paged_range_count(pt, mid) <= target)
            hi = mid;
        else
            lo = mid + 1;
    }
    return lo;
}

// Range c's sequence b and that sequence's first range, or b = -1 when c is
// past the last range.
__device__ __forceinline__ void paged_find_range(const PagedTiles &pt, int lt, int c, int lane,
                                                 int &b, int &first)
{
    b = -1;
    first = 0;
    int base = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (r >= pt.nreg) break;
        const int n = (pt.t[r] + lt - 1) / lt;
        const int incl = wave_incl_scan(n, lane);
        const unsigned long long hit = __ballot(base + incl > c);
        if (hit) {
            const int ln = __ffsll((long long)hit) - 1;
            b = 64 * r + ln;
            first = base + __builtin_amdgcn_readlane(incl - n, ln);
            return;
        }
        base += __builtin_amdgcn_readlane(incl, 63);
    }
}

// Sequence b's first range and range count.
__device__ __forceinline__ void paged_ranges_of(const PagedTiles &pt, int b, int lt, int lane,
                                                int &first, int &count)
{
    int before = 0, mine = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (r >= pt.nreg) break;
        const int n = (pt.t[r] + lt - 1) / lt;
        before += 64 * r + lane < b ? n : 0;
        mine += 64 * r + lane == b ? n : 0;
    }
    first = wave_sum_i32(before);
    count = wave_sum_i32(mine);
}

template <int D, bool OUT_F32, int PPT>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(D >= 256 ? 1 : 2)))
fa_decode_paged_kernel(const Params p, const PagedParams pp)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    constexpr int BN = kDecodeBN;
    using TL = PagedTileLoader<D, BN, PPT>;
    constexpr int TB = TL::TILE_BYTES;
    constexpr int STAGE = 2 * TB;

    constexpr int S = kDecodeStages;
    // D >= 256: separate K and V rings, as in fa_decode_split_kernel
    constexpr int KS = kDecodeKStages256, VS = kDecodeVStages256;
    constexpr int LDS_BYTES = D >= 256 ? (KS + VS) * TB : S * STAGE;
    __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];

    const int lane = threadIdx.x;
    const int col = lane & 31;
    const int half = lane >> 5;

    OperandOffsets<D> off;
    off.init(lane);

    const int item = blockIdx.x;
    int b, g, s, k_begin, k_end;
    if (pp.balanced) {
        // item = (range s, KV head g); the ranges of all sequences in a row
        // Sequence b owns items [first_b Hkv, (first_b + n_b) Hkv): its n_b
        // ranges for each KV head in turn (KV head major, the equal splits'
        // order).  With each KV head's items on other XCDs than in this
        // order, the same ranges streamed 4-8 % slower.
        const PagedTiles pt = paged_tiles(pp, p.B, lane);
        const int lt = paged_range_tiles(pp, pt, p.Hkv);
        if (item < p.B) {
            // the merge's table: sequence `item`'s first range and range count
            int f, n;
            paged_ranges_of(pt, item, lt, lane, f, n);
            if (lane == 0) {
                pp.range_info[2 * item] = f;
                pp.range_info[2 * item + 1] = n;
            }
        }
        int first;
        paged_find_range(pt, lt, item / p.Hkv, lane, b, first);
        if (b < 0) return;                      // past the last range: the whole wave
        const int n_b = max(1, (paged_tiles_of(pt, b) + lt - 1) / lt);
        const int local = item - first * p.Hkv;
        g = local / n_b;
        s = first + local % n_b;                // the range, numbered over all sequences
        // (first <= s by construction; the clamps keep every key index in
        // [0, Sk_b] whatever the range table says)
        const int sk_b = paged_seq_len(pp, b);
        k_begin = min(max(s - first, 0) * lt * BN, sk_b);
        k_end = min(k_begin + lt * BN, sk_b);
    } else {
        s = item % p.num_splits;
        const int bg = item / p.num_splits;
        b = bg / p.Hkv;
        g = bg % p.Hkv;
        const int sk_b = paged_seq_len(pp, b);
        int len = (sk_b + p.num_splits - 1) / p.num_splits;
        len = (len + BN - 1) / BN * BN;
        k_begin = min(s * len, sk_b);
        k_end = min(k_begin + len, sk_b);
    }

    const int rows = p.Sq * p.group;
    const bool valid = col < rows;
    const int qi = valid ? col / p.group : 0;
    const int hq = g * p.group + (valid ? col % p.group : 0);

    const int sk = paged_seq_len(pp, b);
    const int n_tiles = (k_end - k_begin + BN - 1) / BN;

    TL ld;
    ld.setup(p.k + g * D, p.v + g * D, pp.table + (long)b * pp.max_pages, pp.max_pages, k_begin, k_end,
             pp.lg_page, pp.num_pages, ((long)p.Hkv * D) << pp.lg_page, p.Hkv * D * 2, lane);

    bf16x8_t qf[D / 16];
    f32x16_t o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
    float m_ref = kNegInf, l_run = 0.0f, l_rnd = 0.0f;

    const int offk = sk - p.Sq;
    const int lim_lane = p.causal ? qi + offk : 0x7fffffff;
    const int wmin_lim = p.causal ? offk : 0x7fffffff;

    char *const kring = lds, *const vring = lds + KS * TB;
    if constexpr (D >= 256) {
        if (n_tiles > 0) {
            ld.template issue_one<false>(kring, k_begin, 0, lane);
            ld.template issue_one<true>(vring, k_begin, 0, lane);
        }
        if (n_tiles > 1) ld.template issue_one<false>(kring + TB, k_begin + BN, 0, lane);
    } else {
#pragma unroll
        for (int u = 0; u < S - 1; ++u)
            if (u < n_tiles)
                ld.issue(lds + u * STAGE, lds + u * STAGE + TB, k_begin + u * BN, 0, lane);
    }
    load_q<D>(qf, p.q + (((long)b * p.Sq + qi) * p.Hq + hq) * D, half);
    flip_q<D>(qf, p.qflip);
    wait_vmem();   // as in fa_decode_split_kernel: no ring drain per trip
    if constexpr (D >= 256) {
        // one tile per trip over separate K and V rings; the waits and the
        // copy order are those of fa_decode_split_kernel at D = 256
        constexpr int LPT = TL::PER_WAVE;
        int ks = 0, vs = 0;
        for (int n = 0; n < n_tiles; ++n) {
            if (n + 1 < n_tiles)
                __builtin_amdgcn_s_waitcnt((LPT & 15) | ((LPT >> 4) << 14) | 0x0F70);
            else
                wait_vmem();
            __syncthreads();
            if (n + 1 < n_tiles)
                ld.template issue_one<true>(vring + (vs ^ 1) * TB, k_begin + (n + 1) * BN, 0,
                                            lane);
            if (n + 2 < n_tiles) {
                const int k2 = ks + 2 >= KS ? ks + 2 - KS : ks + 2;
                ld.template issue_one<false>(kring + k2 * TB, k_begin + (n + 2) * BN, 0, lane);
            }
            const int key0 = k_begin + n * BN;
            WaveTile<D, BN>::template step<true>(kring + ks * TB, vring + vs * TB, off, qf, o,
                                                 m_ref, l_run, l_rnd, p.c, half, key0, k_end,
                                                 lim_lane);
            ks = ks + 1 == KS ? 0 : ks + 1;
            vs ^= 1;
        }
    } else {
        // S tiles per trip keep every stage offset a compile-time constant
        for (int n = 0; n < n_tiles; n += S) {
#pragma unroll
            for (int u = 0; u < S; ++u)
                if (n + u < n_tiles)
                    decode_step<D, BN, S, TL>(n + u, n_tiles, k_begin, lds, u, ld, lane, k_end,
                                              wmin_lim, off, qf, o, m_ref, l_run, l_rnd, p.c,
                                              half, lim_lane);
        }
    }

    const float l_norm = add_halves(l_rnd);
    if (!pp.balanced && p.num_splits == 1) {
        finish_rows<D, OUT_F32>(o, m_ref, l_run, l_norm, p.c, half, p.o,
                                (((long)b * p.Sq + qi) * p.Hq + hq) * D,
                                p.lse ? p.lse + ((long)b * p.Hq + hq) * p.Sq + qi : nullptr, valid);
    } else {
        // partial rows: [split][B][Hq][Sq], or [range][Hq][Sq] when balanced
        const long prow = pp.balanced ? ((long)s * p.Hq + hq) * p.Sq + qi
                                      : (((long)s * p.B + b) * p.Hq + hq) * p.Sq + qi;
        finish_rows<D, true>(o, m_ref, l_run, l_norm, p.c, half, p.part_o, prow * D,
                             p.part_lse + prow, valid);
    }
#endif
}

// ---------------------------------------------------------------------------
// Merge of split partials, one wave per output row (b, hq, i):
//   M = max_s LSE_s, w_s = exp(LSE_s - M), LSE = M + ln sum_s w_s,
//   O = sum_s w_s O_s / sum_s w_s; splits with LSE_s = -inf weigh 0, and a row
//   whose splits are all -inf gets O = 0, LSE = -inf.
// ---------------------------------------------------------------------------
// Output row `row` from the partials at first, first + stride, ... (ns of them).
template <int D, bool OUT_F32>
__device__ __forceinline__ void merge_row(const Params &p, long row, long first, long stride,
                                          int ns, int lane)
{
    float M = kNegInf;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, p.part_lse[first + s * stride]);
    const float Mu = (M == kNegInf) ? 0.0f : M;

    constexpr int PER = D / 64;                  // head dims per lane
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
    float wsum = 0.0f;
    for (int s = 0; s < ns; ++s) {
        const float ls = p.part_lse[first + s * stride];
        const float w = (ls == kNegInf) ? 0.0f : __expf(ls - Mu);
        wsum += w;
        const float *po = p.part_o + (first + s * stride) * D + lane * PER;
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

template <int D, bool OUT_F32>
__global__ void __launch_bounds__(64) fa_merge_kernel(const Params p)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    const long row = blockIdx.x;                 // (b, hq, i) with i fastest
    const long n_rows = (long)p.B * p.Hq * p.Sq;
    merge_row<D, OUT_F32>(p, row, row, n_rows, p.num_splits, threadIdx.x);
#endif
}

// The merge of the length-balanced paged decode: row (b, hq, i) combines the
// partials of sequence b's ranges, [range][Hq][Sq], which the split kernel
// listed in range_info; a sequence without keys has no range and gets O = 0,
// LSE = -inf.
template <int D, bool OUT_F32>
__global__ void __launch_bounds__(64) fa_merge_paged_kernel(const Params p, const PagedParams pp)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    const int lane = threadIdx.x;
    const long row = blockIdx.x;
    const int i = (int)(row % p.Sq);
    const int hq = (int)((row / p.Sq) % p.Hq);
    const int b = (int)(row / ((long)p.Sq * p.Hq));
    // written by the split kernel's first B items; clamped to the partials
    // the workspace holds
    const int first = min(max(pp.range_info[2 * b], 0), pp.range_cap);
    const int count = min(max(pp.range_info[2 * b + 1], 0), pp.range_cap - first);
    merge_row<D, OUT_F32>(p, row, ((long)first * p.Hq + hq) * p.Sq + i, (long)p.Hq * p.Sq, count,
                          lane);
#endif
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
    p.n_mblocks = 0;
    p.domains = 1;
    p.head_major = 0;
    p.num_splits = L.num_splits;
    p.split_len = L.split_len;
    return p;
}

}  // namespace kern

using namespace kern;

template <int D, int BN, int NW, int NR>
static void launch_prefill_cfg(const Launch &L, const Params &p)
{
    dim3 g(L.grid), blk(NW * 64);
    if constexpr (D == 256) {
        static_assert(BN == 32 && NR == 1, "head dim 256: the pipelined 32-key kernel");
        if (L.o_f32)
            hipLaunchKernelGGL((fa_prefill_pipe_kernel<D, NW, true>), g, blk, 0, L.stream, p);
        else
            hipLaunchKernelGGL((fa_prefill_pipe_kernel<D, NW, false>), g, blk, 0, L.stream, p);
    } else if constexpr (NR == 1) {
        if (L.o_f32)
            hipLaunchKernelGGL((fa_prefill_kernel<D, BN, NW, true>), g, blk, 0, L.stream, p);
        else
            hipLaunchKernelGGL((fa_prefill_kernel<D, BN, NW, false>), g, blk, 0, L.stream, p);
    } else {
        if (L.o_f32)
            hipLaunchKernelGGL((fa_prefill_wide_kernel<D, BN, NW, true>), g, blk, 0, L.stream, p);
        else
            hipLaunchKernelGGL((fa_prefill_wide_kernel<D, BN, NW, false>), g, blk, 0, L.stream,
                               p);
    }
}

template <int D, int NS>
static void launch_prefill_pp(const Launch &L, const Params &p)
{
    dim3 g(L.grid), blk(kPPWaves * 64);
    if (L.o_f32)
        hipLaunchKernelGGL((fa_prefill_pp_kernel<D, NS, true>), g, blk, 0, L.stream, p);
    else
        hipLaunchKernelGGL((fa_prefill_pp_kernel<D, NS, false>), g, blk, 0, L.stream, p);
}

// The compiled prefill tile configurations: head dim, keys per tile, waves
// per workgroup, 32-row column blocks per wave.
struct PrefillCfg {
    int D, bn, nw, nr;
    void (*launch)(const Launch &, const Params &);
};
static const PrefillCfg kPrefillCfgs[] = {
    {128, 64, 8, 1, launch_prefill_cfg<128, 64, 8, 1>},
    {128, 64, 4, 1, launch_prefill_cfg<128, 64, 4, 1>},
    {128, 32, 4, 1, launch_prefill_cfg<128, 32, 4, 1>},
    {128, 32, 8, 1, launch_prefill_cfg<128, 32, 8, 1>},
    {128, 64, 4, 2, launch_prefill_cfg<128, 64, 4, 2>},
    {64, 64, 8, 1, launch_prefill_cfg<64, 64, 8, 1>},
    {64, 64, 4, 1, launch_prefill_cfg<64, 64, 4, 1>},
    {64, 32, 4, 1, launch_prefill_cfg<64, 32, 4, 1>},
    {64, 32, 2, 1, launch_prefill_cfg<64, 32, 2, 1>},
    {128, 32, 2, 1, launch_prefill_cfg<128, 32, 2, 1>},
    {64, 64, 4, 2, launch_prefill_cfg<64, 64, 4, 2>},
    {256, 32, 4, 1, launch_prefill_cfg<256, 32, 4, 1>},
};

static const PrefillCfg *find_prefill_cfg(int D, int bn, int nw, int nr)
{
    for (const PrefillCfg &c : kPrefillCfgs)
        if (c.D == D && c.bn == bn && c.nw == nw && c.nr == nr) return &c;
    return nullptr;
}

bool prefill_cfg_ok(int D, int bn, int nw, int nr) { return find_prefill_cfg(D, bn, nw, nr); }

bool prefill_pp_ok(int D, int stages) { return (D == 64 || D == 128) && (stages == 4 || stages == 5); }

hipError_t launch_prefill(const Launch &L)
{
    if (L.prefill_pp) {
        if (!prefill_pp_ok(L.D, L.prefill_pp)) return hipErrorInvalidValue;
        Params p = make_params(L);
        const int BH = L.B * L.Hq;
        const int bm = 32 * kPPWaves;
        p.n_mblocks = (L.Sq + bm - 1) / bm;
        p.domains = (BH % 8 == 0 && L.grid % 8 == 0) ? 8 : 1;
        p.head_major = L.head_major;
        if (L.D == 128) {
            if (L.prefill_pp == 5) launch_prefill_pp<128, 5>(L, p);
            else launch_prefill_pp<128, 4>(L, p);
        } else {
            if (L.prefill_pp == 5) launch_prefill_pp<64, 5>(L, p);
            else launch_prefill_pp<64, 4>(L, p);
        }
        return hipGetLastError();
    }
    if (L.prefill_pipe) {
        // the pipelined 32-key kernel at head dim 128: 8 waves x 32 rows
        if (L.D != 128 || L.prefill_bn != 32 || L.prefill_nw != 8 || L.prefill_nr != 1)
            return hipErrorInvalidValue;
        Params p = make_params(L);
        const int BH = L.B * L.Hq;
        p.n_mblocks = (L.Sq + 255) / 256;
        p.domains = (BH % 8 == 0 && L.grid % 8 == 0) ? 8 : 1;
        p.head_major = L.head_major;
        dim3 g(L.grid), blk(8 * 64);
        if (L.o_f32)
            hipLaunchKernelGGL((fa_prefill_pipe_kernel<128, 8, true>), g, blk, 0, L.stream, p);
        else
            hipLaunchKernelGGL((fa_prefill_pipe_kernel<128, 8, false>), g, blk, 0, L.stream, p);
        return hipGetLastError();
    }
    const PrefillCfg *cfg = find_prefill_cfg(L.D, L.prefill_bn, L.prefill_nw, L.prefill_nr);
    if (!cfg) return hipErrorInvalidValue;
    Params p = make_params(L);
    const int BH = L.B * L.Hq;
    const int bm = 32 * L.prefill_nw * L.prefill_nr;
    p.n_mblocks = (L.Sq + bm - 1) / bm;
    // one XCD domain per (b, hq) residue class when both counts divide by 8
    p.domains = (BH % 8 == 0 && L.grid % 8 == 0) ? 8 : 1;
    p.head_major = L.head_major;
    cfg->launch(L, p);
    return hipGetLastError();
}

// Calls f(D, OUT_F32) with the call's head dim and output type as
// compile-time constants (std::integral_constant values).
template <class F>
static void with_head_dim(const Launch &L, F &&f)
{
    auto out = [&](auto d) {
        if (L.o_f32)
            f(d, std::true_type{});
        else
            f(d, std::false_type{});
    };
    if (L.D == 256)
        out(std::integral_constant<int, 256>{});
    else if (L.D == 128)
        out(std::integral_constant<int, 128>{});
    else
        out(std::integral_constant<int, 64>{});
}

hipError_t launch_prefill_fp8(const Launch &L, float v_descale)
{
    if (L.D != 128 || (L.prefill_nw != 4 && L.prefill_nw != 8)) return hipErrorInvalidValue;
    Params p = make_params(L);
    const int BH = L.B * L.Hq;
    const int bm = 32 * L.prefill_nw;
    p.n_mblocks = (L.Sq + bm - 1) / bm;
    p.domains = (BH % 8 == 0 && L.grid % 8 == 0) ? 8 : 1;
    p.head_major = L.head_major;
    dim3 g(L.grid), blk(64 * L.prefill_nw);
    auto go = [&](auto nw, auto of) {
        hipLaunchKernelGGL((fa_prefill_fp8_kernel<128, decltype(nw)::value, decltype(of)::value>),
                           g, blk, 0, L.stream, p, v_descale);
    };
    if (L.fp8_pipe) {
        // the pipelined kernel: 8 waves x 32 rows, two waves per SIMD
        if (L.prefill_nw != kFp8PipeWaves) return hipErrorInvalidValue;
        if (L.o_f32)
            hipLaunchKernelGGL((fa_prefill_fp8_pipe_kernel<128, true>), g, blk, 0, L.stream, p,
                               v_descale);
        else
            hipLaunchKernelGGL((fa_prefill_fp8_pipe_kernel<128, false>), g, blk, 0, L.stream, p,
                               v_descale);
        return hipGetLastError();
    }
    if (L.prefill_nw == 8) {
        if (L.o_f32) go(std::integral_constant<int, 8>{}, std::true_type{});
        else go(std::integral_constant<int, 8>{}, std::false_type{});
    } else {
        if (L.o_f32) go(std::integral_constant<int, 4>{}, std::true_type{});
        else go(std::integral_constant<int, 4>{}, std::false_type{});
    }
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdLaunch &L)
{
    if (L.D != 64 && L.D != 128) return hipErrorInvalidValue;
    BwdParams p;
    p.q = static_cast<const uint16_t *>(L.q);
    p.k = static_cast<const uint16_t *>(L.k);
    p.v = static_cast<const uint16_t *>(L.v);
    p.o = static_cast<const uint16_t *>(L.o);
    p.dout = static_cast<const uint16_t *>(L.dout);
    p.lse = L.lse;
    p.ndelta = L.delta;
    p.lse2 = L.delta + (long)L.B * L.Hq * L.Sq;
    p.dq = static_cast<uint16_t *>(L.dq);
    p.dk = static_cast<uint16_t *>(L.dk);
    p.dv = static_cast<uint16_t *>(L.dv);
    p.B = L.B;
    p.Hq = L.Hq;
    p.Hkv = L.Hkv;
    p.Sq = L.Sq;
    p.Sk = L.Sk;
    p.group = L.Hq / L.Hkv;
    p.causal = L.causal;
    p.off = L.Sk - L.Sq;
    p.c = (L.scale < 0.0f ? -L.scale : L.scale) * 1.4426950408889634f;
    p.scale = L.scale;
    p.flip = L.scale < 0.0f ? 0x80008000u : 0u;

    const long rows = (long)L.B * L.Sq * L.Hq;
    dim3 gd((unsigned)((rows + 255) / 256)), bd(256);
    auto by_d = [&](auto d) {
        constexpr int D = decltype(d)::value;
        hipLaunchKernelGGL((fa_bwd_delta_kernel<D>), gd, bd, 0, L.stream, p);
        BwdParams pk = p;
        pk.n_blocks = (L.Sk + kBwdKeysPerWG - 1) / kBwdKeysPerWG;
        hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, kBwdKeysPerWG / 32>), dim3(L.grid_dkdv),
                           dim3(64 * (kBwdKeysPerWG / 32)), 0, L.stream, pk);
        BwdParams pq = p;
        pq.n_blocks = (L.Sq + kBwdRowsPerWG - 1) / kBwdRowsPerWG;
        hipLaunchKernelGGL((fa_bwd_dq_kernel<D, kBwdRowsPerWG / 32>), dim3(L.grid_dq),
                           dim3(64 * (kBwdRowsPerWG / 32)), 0, L.stream, pq);
    };
    if (L.D == 128)
        by_d(std::integral_constant<int, 128>{});
    else
        by_d(std::integral_constant<int, 64>{});
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split partials of the allocation-free entry point (fa_fwd_noalloc): one
// array per GPU the library runs on, held until the process ends.  In host
// code `scratch` only names the symbol; its device address, different on
// every GPU, comes from hipGetSymbolAddress with that GPU current, looked up
// once per device and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices];
}  // namespace

hipError_t static_scratch_ptr(int dev, void **out)
{
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        // the caller has made `dev` the current device
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

static hipError_t launch_merge(const Launch &L, const Params &p)
{
    dim3 gm((unsigned)((long)L.B * L.Hq * L.Sq)), blk(64);
    with_head_dim(L, [&](auto d, auto of) {
        hipLaunchKernelGGL((fa_merge_kernel<decltype(d)::value, decltype(of)::value>), gm, blk,
                           0, L.stream, p);
    });
    return hipGetLastError();
}

hipError_t launch_decode(const Launch &L)
{
    Params p = make_params(L);
    dim3 g(L.B * L.Hkv * L.num_splits), blk(64);
    with_head_dim(L, [&](auto d, auto of) {
        hipLaunchKernelGGL((fa_decode_split_kernel<decltype(d)::value, decltype(of)::value>), g,
                           blk, 0, L.stream, p);
    });
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || L.num_splits == 1) return e;
    return launch_merge(L, p);
}

template <int PPT>
static void launch_paged_cfg(const Launch &L, const Params &p, const PagedParams &pp, dim3 g)
{
    dim3 blk(64);
    with_head_dim(L, [&](auto d, auto of) {
        hipLaunchKernelGGL((fa_decode_paged_kernel<decltype(d)::value, decltype(of)::value, PPT>),
                           g, blk, 0, L.stream, p, pp);
    });
}

hipError_t launch_decode_paged(const Launch &L, const PagedLaunch &P)
{
    Params p = make_params(L);
    PagedParams pp;
    pp.table = P.table;
    pp.seq_lens = P.seq_lens;
    pp.max_pages = P.max_pages;
    pp.num_pages = P.num_pages;
    pp.lg_page = 0;
    while ((1 << pp.lg_page) < P.page_size) ++pp.lg_page;
    pp.balanced = P.balanced;
    pp.slots = P.slots;
    pp.range_cap = P.range_cap;
    pp.len_min = P.len_min;
    pp.len_max = P.len_max;
    pp.range_info = P.balanced ? reinterpret_cast<int *>(L.part_lse + (size_t)P.range_cap * L.Hq * L.Sq)
                               : nullptr;
    dim3 g(P.balanced ? L.Hkv * P.range_cap : L.B * L.Hkv * L.num_splits);
    // pages per 32-key tile: 1, or 2 for 16-key pages
    if (P.page_size >= kDecodeBN)
        launch_paged_cfg<1>(L, p, pp, g);
    else
        launch_paged_cfg<kDecodeBN / 16>(L, p, pp, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (P.balanced) {
        dim3 gm((unsigned)((long)L.B * L.Hq * L.Sq)), blk(64);
        with_head_dim(L, [&](auto d, auto of) {
            hipLaunchKernelGGL((fa_merge_paged_kernel<decltype(d)::value, decltype(of)::value>),
                               gm, blk, 0, L.stream, p, pp);
        });
        return hipGetLastError();
    }
    if (L.num_splits == 1) return e;
    return launch_merge(L, p);
}

}  // namespace fa
