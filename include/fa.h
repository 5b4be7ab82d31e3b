/*
 * fa.h -- C ABI of the MI355X (gfx950) fused attention forward library.
 *
 * Operation.  For every batch b, query head hq, query row i:
 *
 *   O[b,i,hq,:] = softmax_j( scale * q[b,i,hq,:] . k[b,j,g,:] )  V[b,j,g,:]
 *   LSE[b,hq,i] = ln sum_j exp( scale * q[b,i,hq,:] . k[b,j,g,:] )
 *
 * over the allowed keys j, with g = hq / (Hq / Hkv).  This is the fused
 * attention forward whose tiled SM80 and SM90 main loops are laid out in
 * "SM80 内核实现对比" (Inference Cookbook, FlashAttention), sections 4.1 and
 * 5.2: Q K^T, online softmax, then P V, with S and P kept on chip.  The
 * softmax components (row max, exp, row sum, rescale, causal mask) are the ones
 * listed in "从 Volta/Turing、Ampere、Ada 到 Hopper：硬件、PTX 与 Kernel 编程范式
 * 演进", section "Attention 的瓶颈会在 Tensor Core 与 CUDA Core 之间迁移".  The
 * pages give no interface, no layout and no LSE; those are this library's
 * choices:
 *
 *   layout   q, o : [B][Sq][Hq][D]   k, v : [B][Sk][Hkv][D]   (D innermost,
 *            fully contiguous, row-major)      lse : [B][Hq][Sq] float32
 *   causal   key j is allowed for query i iff j <= i + (Sk - Sq); a row with
 *            no allowed key gets O = 0 and LSE = -inf
 *   dtypes   q, k, v bfloat16; o bfloat16 (round to nearest even) or float32;
 *            all arithmetic accumulates in float32
 *
 * Conventions shared by every call:
 *   - All pointers except `workspace` of fa_fwd_ex are device pointers owned
 *     by the caller; the library neither frees nor retains them.  Each must be
 *     16-byte aligned.  `lse` may be NULL (then no LSE is written).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  Nothing inside synchronises the host.  All launches of one call
 *     go to that one stream, in order.
 *   - Results are deterministic: repeated calls with the same arguments give
 *     bit-identical outputs (no floating-point atomics).
 *   - Argument checks run before any HIP call and return synchronously.
 *   - Every non-OK status leaves a message for fa_last_error() in the calling
 *     thread.  No call throws, aborts or prints (unless FA_LOG=1 is set, which
 *     prints the chosen plan to stderr).
 *   - Thread-safe: calls may come from several host threads.  The
 *     library-owned split workspace (see fa_fwd_ex) is one buffer per device,
 *     shared by every call on that device: split-path calls whose kernels may
 *     overlap in time (different streams) must each pass their own workspace.
 *     Growing that buffer frees the old one with hipFree, which waits for the
 *     device; this is the only point where a call can block the host.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1, /* NULL q/k/v/o, a dimension < 1, Hq % Hkv != 0,
                               non-finite scale, bad workspace size          */
    FA_ERR_UNSUPPORTED = 2, /* D not in {64, 128, 256}, pointer not 16-B aligned,
                               device not gfx950, split request the split
                               path cannot serve, sizes beyond 32-bit indexing */
    FA_ERR_NOMEM = 3,       /* the library-owned workspace could not be
                               allocated                                     */
    FA_ERR_HIP = 4          /* a HIP call failed; fa_last_error() has its text */
} fa_status;

typedef enum { FA_DTYPE_BF16 = 0, FA_DTYPE_F32 = 1 } fa_dtype;

/*
 * fa_fwd -- attention forward, bf16 O.  Same as
 * fa_fwd_ex(..., FA_DTYPE_BF16, 0, NULL, 0).
 *
 * q   [B][Sq][Hq][D]  bf16, device     k, v  [B][Sk][Hkv][D]  bf16, device
 * o   [B][Sq][Hq][D]  bf16, device     lse   [B][Hq][Sq] float32, device or NULL
 * causal: 0 or 1.  scale: any finite float applied to the raw dot products
 * (negative and zero included).
 */
fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                 int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale,
                 hipStream_t stream);

/*
 * fa_fwd_ex -- as fa_fwd, plus:
 *   o_dtype      FA_DTYPE_BF16 or FA_DTYPE_F32 (o then holds float32).
 *   num_splits   0 = let the library choose.  >= 1 forces the split-key path:
 *                the key range is cut into num_splits contiguous pieces, each
 *                piece produces a partial (O_s, LSE_s), and a merge pass
 *                combines them by log-sum-exp weights.  The split path serves
 *                problems whose Sq * (Hq / Hkv) query rows per KV head fit one
 *                64-lane wave's tile (<= 32); otherwise FA_ERR_UNSUPPORTED.
 *                num_splits is clamped to ceil(Sk / 32).  The split-key
 *                decomposition and merge are not on the pages; they follow
 *                from the log-sum-exp definition above.
 *   workspace    device memory for the split partials, or NULL for a
 *                library-owned buffer (allocated on first need per device,
 *                grown on demand, kept until fa_release_workspace).
 *   workspace_bytes  size of `workspace`; must be >= fa_workspace_size(...)
 *                of the same problem when `workspace` is not NULL.
 */
fa_status fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                    int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale,
                    hipStream_t stream, fa_dtype o_dtype, int num_splits, void *workspace,
                    size_t workspace_bytes);

/*
 * fa_fwd_noalloc -- fa_fwd_ex for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and arguments, without a workspace.  The
 * split partials go to a static device array of 16 MiB that the library
 * holds on every GPU it runs on until the process ends; a plan that needs
 * more than that (fa_workspace_size of the same problem) returns
 * FA_ERR_UNSUPPORTED, and the prefill path needs none.  The call allocates
 * nothing (no hipMalloc, no library allocation); its first call on a device
 * looks up that device's array address once.  Every call on one GPU shares
 * that GPU's array and leaves its contents behind (no call needs them
 * cleared): calls on one GPU whose kernels may overlap in time, i.e. on
 * different streams without ordering, race and must not be made.  Other
 * arguments, statuses and asynchrony as for fa_fwd_ex.
 */
fa_status fa_fwd_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                         int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale,
                         hipStream_t stream, fa_dtype o_dtype, int num_splits);

/*
 * fa_workspace_size -- bytes of split workspace the call with these sizes and
 * this num_splits (0 = automatic) needs; 0 when it takes the single-pass path.
 * Hkv is an argument because the automatic split count depends on the number
 * of (batch, KV head) pairs.  Host arithmetic plus a one-time query of the
 * current device's compute-unit count (a device property: nothing is
 * launched or allocated), so the size asked for before any call equals what
 * fa_fwd_ex then needs on that device; with no usable device it plans for
 * 256 compute units.  Returns 0 for invalid sizes.
 */
size_t fa_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int D, int num_splits);

/*
 * fa_plan -- which kernels a call with these sizes would launch.  Host
 * arithmetic plus the one-time device property query of fa_workspace_size.
 * Fills *out; returns FA_ERR_INVALID_ARG / FA_ERR_UNSUPPORTED as fa_fwd_ex would.
 */
typedef struct {
    int path;            /* 0 = prefill (single pass), 1 = split-key decode + merge,
                            2 = paged split-key decode + merge (fa_plan_paged)    */
    int num_splits;      /* 1 for the prefill path                                */
    int block_m;         /* query rows per workgroup tile                          */
    int block_n;         /* keys per K/V tile                                      */
    int grid;            /* workgroups of the main kernel                          */
    int work_items;      /* tiles of work the grid walks                           */
    size_t workspace_bytes;
    int waves;           /* waves per workgroup of the main kernel                 */
    int rows_per_wave;   /* prefill: query rows per wave (32, or 64 for the kernel
                            that holds two 32-row column blocks per wave); 0 for
                            the split-key path                                    */
} fa_plan_info;

fa_status fa_plan(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int num_splits,
                  fa_plan_info *out);

/*
 * fa_fwd_paged -- the same attention forward over a paged K/V cache, with a
 * key count per sequence (decode, and short multi-token queries).
 *
 * The pages list paged K/V only as a loading mode of the SM80 and SM90
 * kernels ("SM80 内核实现对比", section 7.3, the PagedKV row: both fetch it
 * with cp.async); the layout and the meaning below are this library's:
 *
 *   q, o         [B][Sq][Hq][D] as for fa_fwd (o bf16 or f32 per o_dtype);
 *                lse [B][Hq][Sq] float32 or NULL
 *   k_cache,     [num_pages][page_size][Hkv][D] bf16, device: num_pages
 *   v_cache      pages of page_size keys each
 *   block_table  [B][max_pages] int32, device: key j of sequence b is slot
 *                j % page_size of cache page block_table[b][j / page_size]
 *   seq_lens     [B] int32, device: Sk_b, the keys of sequence b; read by the
 *                kernels (no host synchronisation) and clamped to
 *                [0, max_pages * page_size]
 *
 * Sequence b is then exactly fa_fwd over its first Sk_b keys: causal allows
 * key j for query i iff j <= i + Sk_b - Sq, and a row with no allowed key
 * (Sk_b = 0, say) gets O = 0 and LSE = -inf.
 *
 * page_size: a power of two >= 16.  Sq * Hq / Hkv <= 32 (the split-key
 * decode's tile), else FA_ERR_UNSUPPORTED.
 * num_splits: 0 = automatic.  For B <= 256 the automatic cut is length
 * balanced: every sequence's keys are cut into ranges of one common length,
 * chosen on the device from seq_lens (the shortest multiple of 32 keys, at
 * least 128, for which the (range, KV head) work items fit the GPU's resident
 * decode waves in one round), so that a long sequence gets more ranges than a
 * short one.  Otherwise (num_splits >= 1, or B > 256) each sequence's keys
 * are cut into num_splits equal ranges (multiples of 32 keys); it is raised if
 * needed so that one range spans at most 256 pages.  The result depends on
 * the cut only through rounding (the partial results are merged by their
 * log-sum-exp).
 * workspace / workspace_bytes: as for fa_fwd_ex, sized by fa_plan_paged's
 * workspace_bytes.  Only row b of the block table is read (entries within
 * [0, max_pages)), and only the entries of pages below Sk_b are used.
 * An entry outside [0, num_pages) reads as zero keys and values: results for
 * that sequence are then meaningless, but no memory outside the caches is
 * touched.
 */
fa_status fa_fwd_paged(const void *q, const void *k_cache, const void *v_cache,
                       const int *block_table, const int *seq_lens, void *o, float *lse, int B,
                       int Hq, int Hkv, int Sq, int D, int num_pages, int page_size,
                       int max_pages, int causal, float scale, hipStream_t stream,
                       fa_dtype o_dtype, int num_splits, void *workspace, size_t workspace_bytes);

/*
 * fa_plan_paged -- the launch fa_fwd_paged would make (path 2): splits per
 * sequence (0 for the length-balanced cut, decided on the device), grid,
 * workspace bytes.  Host arithmetic, like fa_plan.
 */
fa_status fa_plan_paged(int B, int Hq, int Hkv, int Sq, int D, int num_pages, int page_size,
                        int max_pages, int num_splits, fa_plan_info *out);

/*
 * fa_fwd_fp8 -- the attention forward on OCP FP8 E4M3 inputs with per-tensor
 * descale factors.  The pages list FP8 only as a capability of the SM90
 * kernel ("SM80 内核实现对比", section 7.3, the FP8 row); the convention is
 * this library's, the usual per-tensor one: the real inputs are
 * q_descale * q, k_descale * k, v_descale * v, and the result is fa_fwd's on
 * those values:
 *
 *   q [B][Sq][Hq][D], k, v [B][Sk][Hkv][D]: E4M3 codes, one byte each, device
 *   o [B][Sq][Hq][D] bf16 or f32 (o_dtype), lse [B][Hq][Sq] f32 or NULL
 *
 * Scores are formed exactly from the codes (products and sums in fp32) and
 * scaled by scale * q_descale * k_descale; P is rounded to E4M3 for the P V
 * product and O is normalised by the sum of the rounded P; the LSE uses the
 * unrounded fp32 P.  D = 128 only (else FA_ERR_UNSUPPORTED); descales must be
 * finite and > 0 (else FA_ERR_INVALID_ARG).  Layout, causal convention,
 * alignment, asynchrony and errors as for fa_fwd; no workspace.
 */
fa_status fa_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                     int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale,
                     float q_descale, float k_descale, float v_descale, hipStream_t stream,
                     fa_dtype o_dtype);

/*
 * fa_bwd -- gradients of the attention forward: dq, dk, dv from q, k, v, the
 * forward's o and lse, and the upstream gradient dout.  The pages list the
 * backward pass only by a page title, so it follows from the forward's
 * mathematics: with P = softmax(scale q k^T [+ causal mask]) (recomputed from
 * lse), delta_i = sum_d dout_id o_id,
 *   dv = P^T dout,  dS = P (dout v^T - delta),  dq = scale dS k,
 *   dk = scale dS^T q,
 * with the query heads of a KV head adding their dk and dv.
 *
 *   q, o, dout, dq  [B][Sq][Hq][D] bf16     k, v, dk, dv  [B][Sk][Hkv][D] bf16
 *   lse             [B][Hq][Sq] float32 (as fa_fwd wrote it)
 *
 * D = 64 or 128.  Every output element is written by one wave (no atomics):
 * results are deterministic.  workspace: device memory of
 * fa_bwd_workspace_size() bytes (delta and LSE * log2 e), or NULL for the library-owned
 * buffer (shared with fa_fwd_ex's split workspace, same rules).  Rows with no
 * allowed key contribute nothing.  Asynchrony, alignment and errors as for
 * fa_fwd.
 */
fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                 const float *lse, void *dq, void *dk, void *dv, int B, int Hq, int Hkv, int Sq,
                 int Sk, int D, int causal, float scale, hipStream_t stream, void *workspace,
                 size_t workspace_bytes);

/* fa_bwd_workspace_size -- bytes of workspace fa_bwd needs (2 * B * Hq * Sq
 * floats: delta and the LSE in base 2); 0 for invalid sizes.  Pure host
 * arithmetic. */
size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Sk, int D);

/* fa_last_error -- message for the last non-OK status of this host thread
 * ("" if none).  The pointer stays valid until the next call on this thread. */
const char *fa_last_error(void);

/* fa_release_workspace -- frees every library-owned workspace (all devices).
 * The caller must make sure no kernel still uses it (synchronise first). */
fa_status fa_release_workspace(void);

/* fa_version -- major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
