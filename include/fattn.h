/*
 * libfattn -- exact tiled (Flash) attention for AMD Instinct MI355X (gfx950).
 *
 * The operation.  For every batch b, query head h and query row i:
 *
 *     s_ij   = scale * q[b,h,i,:] . k[b,g,j,:]      g = h / (H / Hkv)
 *     visible(i,j) = !causal || j <= i
 *     O[b,h,i,:] = sum_j softmax_j(s_i.)[visible] * v[b,g,j,:]
 *     LSE[b,h,i] = ln sum_{visible j} exp(s_ij)
 *
 * This is attention written out as score, softmax and weighted average
 * ("LLM Architecture Refresh [3]: Flash Attention Is Exact", section 1; the
 * stable softmax of section 2; the causal mask of section 5).  The forward
 * computes it tile by tile with a running max, running sum and unnormalised
 * output per query row, rescaled whenever a later tile raises the max ("How
 * FlashAttention Uses Tiling", "The Running Statistics"; the same page 3,
 * section 4), skips key tiles that lie wholly in the future of a causal
 * query tile (section 7), and never writes the N x N score matrix to memory.
 * The backward recomputes the probabilities from Q, K, V and the saved LSE
 * (section 8) instead of storing them.
 *
 * Layout (all tensors dense and row-major, no strides):
 *     q, o, dO, dq      [B, H,   N, d]
 *     k, v, dk, dv      [B, Hkv, N, d]
 *     lse               [B, H,   N]      float32, natural log, scaled-score units
 * Query head h reads key/value head h / (H / Hkv); H must be a multiple of
 * Hkv.  Causal masking is square: key j is visible to query i iff j <= i.
 *
 * Ownership and execution.  Every pointer is a device pointer owned by the
 * caller.  The library allocates nothing, never synchronises, and enqueues
 * its kernels on `stream` (NULL = the default stream) in order; a call returns
 * as soon as the work is enqueued.  Faults during execution surface at the
 * caller's next synchronisation.  All calls are thread-safe; the only global
 * state is fa_bwd_noalloc's per-GPU scratch (see there).
 *
 * Errors.  Arguments are validated before anything is launched; on a non-zero
 * return nothing was enqueued and no output was touched:
 *     FA_ERR_INVALID_ARG  null pointer, negative size, H, Hkv or d <= 0,
 *                         H % Hkv != 0, non-finite scale, a pointer not aligned
 *                         to 16 bytes (4 for lse), an output overlapping an
 *                         input, sizes whose index space exceeds 2^62 or
 *                         whose row count B*H*N exceeds 2^31 - 1, or (the bf16
 *                         and fp8 forwards, the backward) one head's slab of
 *                         (N + 64) * d elements exceeding 2^31 - 1 bytes
 *                         (the last tile addresses up to 64 rows past N);
 *     FA_ERR_UNSUPPORTED  a head dimension other than 64 or 128;
 *     FA_ERR_HIP          the HIP runtime refused the launch;
 *     FA_ERR_TOO_LARGE    (fa_bwd_noalloc only) the problem exceeds its fixed
 *                         scratch.
 * B == 0 or N == 0 is an empty problem: FA_OK, nothing is read, written or
 * launched, and the pointers may be NULL.
 */
#ifndef FATTN_H
#define FATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = -1,
    FA_ERR_UNSUPPORTED = -2,
    FA_ERR_HIP = -3,
    FA_ERR_TOO_LARGE = -4
};

/*
 * Forward, bf16 storage.  q, k, v, o are bf16 (IEEE binary16-brain, raw
 * 16-bit patterns); products accumulate in fp32 on the matrix cores; the
 * running max/sum/rescale are fp32; o is rounded to bf16 with
 * round-to-nearest-even; lse is fp32.  d must be 64 or 128.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Hkv, int N, int d, int causal, float scale,
           hipStream_t stream);

/*
 * Local (sliding-window) causal forward, bf16 storage: query i sees only the
 * keys i - window + 1 .. i.  This is the approximation that "LLM Architecture
 * Refresh [3]: Flash Attention Is Exact", section 5, contrasts with exact
 * attention; key tiles wholly before every row's window are skipped like the
 * future tiles of causal attention (section 7).  Same layout, precision and
 * errors as fa_fwd, plus FA_ERR_INVALID_ARG for window < 1 (checked after the
 * empty-problem test).  window >= N gives exactly fa_fwd with causal = 1.
 */
int fa_fwd_local(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int Hkv, int N, int d, int window, float scale,
                 hipStream_t stream);

/*
 * FP8 forward: q, k, v hold OCP e4m3 codes (one byte per element, same
 * [B, H, N, d] / [B, Hkv, N, d] layouts) whose values are descale_q * e4m3(q)
 * and likewise for k and v (per-tensor scales, each finite and > 0); o is
 * bf16 and lse fp32 as in fa_fwd, for the scores scale * q_i . k_j of those
 * values.  Both products run on the fp8 matrix cores with fp32 accumulation;
 * the attention weights are rounded to e4m3 before they multiply V (the
 * low-precision variant "LLM Architecture Refresh [3]: Flash Attention Is
 * Exact", section 8, credits to FlashAttention-3).  With e_i the largest
 * score error of row i (the fp8 matrix cores sum each 64-term step within
 * 2^-11 of the sum of |q_ic k_jc|), the extra error is bounded elementwise by
 * (2^-4 + 2 e_i) (P|V|)_ic + 2^-16 sum_j |v_jc| plus the bf16 rounding of O,
 * and that of lse by e_i (no fp8 rounding of the weights reaches lse).
 * The 16-byte alignment rule
 * applies to q, k, v, o; errors as fa_fwd, plus FA_ERR_INVALID_ARG for a
 * descale that is not finite and positive.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Hkv, int N, int d, int causal, float scale,
               float descale_q, float descale_k, float descale_v, hipStream_t stream);

/*
 * Forward, fp32 storage and fp32 arithmetic throughout: the same exact
 * attention as fa_fwd ("LLM Architecture Refresh [3]: Flash Attention Is
 * Exact", section 4, the tiled loop; "How FlashAttention Uses Tiling",
 * "The Running Statistics"), for single-precision inputs.  Same layout,
 * ownership and errors as fa_fwd.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int Hkv, int N, int d, int causal, float scale,
               hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes (the per-row
 * D_i = sum_j P_ij dP_ij terms, fp32 [B, H, N], rounded up to 256 bytes).
 * Returns 0 for an empty problem and for invalid sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int Hkv, int N, int d);

/*
 * Backward with recomputation ("LLM Architecture Refresh [3]: Flash
 * Attention Is Exact", section 8: the probabilities are recomputed from Q, K,
 * V and the saved statistics rather than stored), bf16 storage.  Inputs q, k,
 * v, o (the output of fa_fwd), lse (from fa_fwd) and dO; outputs dq
 * [B,H,N,d], dk and dv [B,Hkv,N,d], all bf16 except lse.  The gradient of
 * sum(O * dO):
 *     P_ij  = exp(s_ij - LSE_i)           dP_ij = dO_i . v_j
 *     D_i   = sum_j P_ij dP_ij            dS_ij = P_ij (dP_ij - D_i)
 *     dV_j  = sum_i P_ij dO_i             dQ_i  = scale sum_j dS_ij k_j
 *                                         dK_j  = scale sum_i dS_ij q_i
 * with dK, dV of a key/value head summed over the query heads that read it.
 * D_i equals dO_i . O_i for the exact output; it is recomputed in fp32 from
 * P and dP because the bf16-rounded o would dominate the gradient error, so
 * `o` is validated (non-null, aligned, no overlap with outputs) but not read.
 * `workspace` is caller-owned device memory of at least
 * fa_bwd_workspace_bytes(...) bytes, 16-byte aligned; its contents on entry
 * are ignored.  The result is deterministic (no atomics).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dO, void* dq, void* dk, void* dv, void* workspace,
           int B, int H, int Hkv, int N, int d, int causal, float scale,
           hipStream_t stream);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same operation, layouts, precision and result as
 * fa_bwd (bitwise: the same kernels run); the per-row D terms live in a fixed
 * 16 MiB scratch array that the library holds on each GPU it runs on until
 * the process ends, so B*H*N may be at most 2^22 (4194304) rows, else
 * FA_ERR_TOO_LARGE is returned before anything is launched.  No call
 * allocates or frees memory.  Every call on one GPU shares that GPU's scratch:
 * calls that overlap in time on one GPU (different streams, or different host
 * threads) race and give undefined results; calls ordered on one stream are
 * safe.  The scratch's device address is looked up on the first call on each
 * device (the device that runs `stream`); a failure there is FA_ERR_HIP.
 * Errors otherwise as fa_bwd.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv,
                   int B, int H, int Hkv, int N, int d, int causal, float scale,
                   hipStream_t stream);

/*
 * Device counters of the bf16 forward (fa_fwd, fa_fwd_local), for checking
 * the tile schedule and the rescale rule against a host model: the tile
 * skipping of "LLM Architecture Refresh [3]: Flash Attention Is Exact",
 * section 7, and the counters its section 8 keeps.  Only a library built with
 * the counters (libfattn_counters.so, build option FATTN_DEVICE_COUNTERS)
 * keeps them; the normal library returns FA_ERR_UNSUPPORTED.  A tile is one
 * wave's 32 query rows against one 64-key tile.  out[0..3] receive the totals
 * since the last reset: tiles computed; tiles skipped (key tiles of the
 * sequence a row block never computes); computed tiles that were masked
 * (diagonal, window edge or sequence end); reference raises (a row block's
 * running max moved after its first tile, rebasing l and O).  Synchronises
 * with the device; reset != 0 zeroes the counters afterwards.  out must hold
 * 4 values (FA_ERR_INVALID_ARG when NULL).
 */
int fa_debug_counters(unsigned long long* out, int reset);

/* Static, human-readable name of a status code (never NULL). */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FATTN_H */
