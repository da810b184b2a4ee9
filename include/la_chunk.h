/*
 * la_chunk.h -- C ABI of the MI355X (gfx950) chunked causal linear attention library.
 *
 * The operation ("Fractus-1B training optimization", section 1, Bottleneck #1,
 * and section 2, Opt 2): for each of G independent groups (batch x levels x
 * heads flattened, section 1 "Diagnosis") and a chunk of C tokens with head
 * dimension D, given positive features q_t, k_t (the caller has already applied
 * its feature map), values v_t and a carried state (S_in, z_in),
 *
 *     S_t = S_in + sum_{j<=t} k_j v_j^T      z_t = z_in + sum_{j<=t} k_j      (inclusive of token t)
 *     o_t = (S_t^T q_t) / (q_t . z_t)
 *     S_out = S_C,  z_out = z_C.
 *
 * The forward is computed in the blocked ("chunked") form of section 2, Opt 2:
 * blocks of `block` tokens, a masked block x block score matrix for the block's
 * own tokens plus a term against the running state (S_run, z_run) read before
 * the block updates it; the C mod block tokens left at the end (the ragged
 * tail) take the exact per-token cumsum form.  The backward is the reverse
 * scan the same page names (the gradient of a prefix sum is a suffix sum); it
 * recomputes the forward from its inputs and takes no saved activations.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer (hipMalloc'd or equivalent),
 *     row-major, contiguous, 16-byte aligned.  The caller allocates and owns all
 *     buffers; the library allocates nothing and is reentrant.  The only state
 *     it keeps between calls is a pending timing request (la_time_next_launch),
 *     per calling thread.
 *   - Token tensors q, k, v, o, dO, dq, dk, dv are [G][C][D] in the element type
 *     `dt` (fp32 or bf16).  The state S (and dS) is [G][D][D] fp32 with S[p][c]:
 *     p indexes the key feature, c the value feature; z (and dz) is [G][D] fp32.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued on
 *     it and the call returns at once; the library never synchronises the
 *     device.  Calls on one stream run in stream order.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is launched and a status other than LA_OK is returned.
 *     Nothing is printed, thrown or exited across this boundary.
 *   - Preconditions NOT checked on the device: q_t . z_t > 0 for every token
 *     (true for positive features: q, k > 0 elementwise and z_in >= 0), and
 *     finite inputs.  No epsilon is added to the denominator.
 *   - Supported: D in {64, 128}, block 64 (or 1 for the chunk calls), G >= 1,
 *     1 <= C, and one group's chunk plus 256 tokens below 2 GiB
 *     ((C + 256) * D * element size < 2^31: the kernels address a chunk with
 *     32-bit byte offsets).  The backward additionally needs C <= LA_BWD_MAX_C.
 *     Anything else returns LA_ERR_UNSUPPORTED.
 */
#ifndef LA_CHUNK_H
#define LA_CHUNK_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_ABI_VERSION 6
#define LA_BWD_MAX_C 2048
/* Longest sequences (tokens per group) of the sequence entry points, D = 64 and D = 128:
 * the lengths at which their results are verified to the parity tolerance against an fp64
 * reference from a zero initial carry (the hardest case for the backward, which recovers
 * the early states from the final carry). */
#define LA_SEQ_D64_MAX_T 1048576
#define LA_SEQ_D128_MAX_T 16384

typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

/* Feature map the sequence entry points may apply to q and k themselves. */
typedef enum {
    LA_FEATURE_NONE = 0,  /* q, k are the positive features */
    LA_FEATURE_ELU1 = 1   /* q, k are raw inputs x; the op uses phi(x) = elu(x) + 1 (alpha = 1) */
} la_feature;

typedef enum {
    LA_OK = 0,
    LA_ERR_INVALID = 1,     /* NULL required pointer, G < 1, C < 1, half-given carry, size overflow */
    LA_ERR_UNSUPPORTED = 2, /* D, block, dtype or C outside the supported set */
    LA_ERR_ALIGN = 3,       /* a tensor pointer is not 16-byte aligned */
    LA_ERR_ALIAS = 4,       /* an output overlaps an input or another output */
    LA_ERR_LAUNCH = 5       /* the HIP runtime rejected the kernel launch */
} la_status;

/*
 * Forward over one chunk.
 *   q, k, v  : [G][C][D] dt, inputs.  q and k are positive features (or, with
 *              feature = LA_FEATURE_ELU1, the raw inputs x of the map phi).
 *   S_in     : [G][D][D] fp32 carried state, or NULL (zero state).
 *   z_in     : [G][D]    fp32 carried normaliser, or NULL.  S_in and z_in are
 *              both NULL or both non-NULL.
 *   o        : [G][C][D] dt, output o_t.
 *   S_out    : [G][D][D] fp32, output state after the chunk (S_C).
 *   z_out    : [G][D]    fp32, output normaliser after the chunk (z_C).
 *   block    : 64: the blocked ("chunked") form of section 2, Opt 2 (64-token
 *              blocks, the ragged tail token by token);
 *              1: the cumsum form of the same section (Opt 1 names it among the
 *              selectable forms): the exact per-token recurrence over the whole
 *              chunk, in fp32 arithmetic, no blocking.  Both compute the same
 *              function; they differ only in summation order.
 *   feature  : LA_FEATURE_NONE, or LA_FEATURE_ELU1: q and k hold raw inputs x and
 *              the op runs on phi(x) = elu(x) + 1 computed in fp32 and rounded to
 *              the element type as the inputs are loaded (as in la_seq_fwd).  With
 *              the map, bf16 chunks of 128 tokens at D = 64 and bf16 chunks at D = 128
 *              run their blocked kernels; every other shape runs the per-token form.
 * bf16 at D = 128 (block 64, C up to LA_SEQ_D128_MAX_T) runs la_seq_fwd's kernel over
 * a one-chunk sequence: a ragged end is a masked 64-token block there, not the
 * token-by-token tail (the same function in another summation order).
 * S_out may not alias S_in: the call is pure (the carry goes in, a new carry
 * comes out), so chaining chunks ping-pongs two state buffers.  A feature
 * outside la_feature is LA_ERR_INVALID.
 */
la_status la_chunk_fwd(const void *q, const void *k, const void *v,
                       const float *S_in, const float *z_in,
                       void *o, float *S_out, float *z_out,
                       int G, int C, int D, int block, la_feature feature, la_dtype dt, void *stream);

/*
 * Backward over one chunk, for the loss
 *     L = sum_t <dO_t, o_t> + <dS_out, S_out> + dz_out . z_out.
 *   q, k, v, S_in, z_in : exactly the inputs of the forward call (S_in/z_in may
 *                         be NULL together, meaning a zero carry).
 *   dO       : [G][C][D] dt, gradient of o.
 *   dS_out   : [G][D][D] fp32 gradient of S_out (from the next chunk), or NULL.
 *   dz_out   : [G][D]    fp32 gradient of z_out, or NULL; NULL together with dS_out
 *              (both NULL = zero).
 *   dq,dk,dv : [G][C][D] dt, outputs.
 *   dS_in    : [G][D][D] fp32 output, gradient of S_in (pass it as the previous
 *              chunk's dS_out when chaining).
 *   dz_in    : [G][D]    fp32 output, gradient of z_in.
 *   block, feature : as in the forward call.  With LA_FEATURE_ELU1, dq and dk are
 *              the gradients with respect to the raw inputs: dq phi'(x_q), dk phi'(x_k),
 *              phi'(x) = 1 for x > 0 and e^x otherwise (taken as min(1, phi)).
 * With a NULL carry, dS_in/dz_in still receive the gradient with respect to a
 * zero carry.  fp32 elements at D == 128 run the per-token form whatever the
 * block (the blocked form's fp32 tiles of that size exceed the local memory);
 * its results agree with the blocked form's to fp32 rounding.  bf16 at D == 128
 * (block 64) runs la_seq_bwd's walk over the chunk's 64-token blocks, last first,
 * after building the carry after the chunk from S_in, z_in in the same launch.
 */
la_status la_chunk_bwd(const void *q, const void *k, const void *v,
                       const float *S_in, const float *z_in,
                       const void *dO, const float *dS_out, const float *dz_out,
                       void *dq, void *dk, void *dv, float *dS_in, float *dz_in,
                       int G, int C, int D, int block, la_feature feature, la_dtype dt, void *stream);

/*
 * Forward over a whole sequence: n = T / chunk consecutive chunks per group, in order,
 * with the carry passed from each chunk to the next on chip (the carry across
 * consecutive chunks of "Fractus-1B training optimization", section 2).  The result is
 * that of n chained la_chunk_fwd calls over the chunks up to fp32 rounding (the state
 * S and the normaliser z carry their compensation terms from chunk to chunk instead of
 * being rounded at each boundary), but no carry between chunks goes through memory and
 * the whole sequence is one launch.
 *   q, k, v  : [G][T][D] dt, inputs; chunk c of a group is its tokens
 *              c*chunk .. (c+1)*chunk - 1.
 *   S_in     : [G][D][D] fp32 carry before the first chunk, or NULL (zero state).
 *   z_in     : [G][D]    fp32, or NULL; NULL together with S_in.
 *   o        : [G][T][D] dt, output.
 *   S_out    : [G][D][D] fp32, state after the last chunk.
 *   z_out    : [G][D]    fp32, normaliser after the last chunk.
 *   S_res    : [G][D][D] fp32 output, or NULL: the remainder of the final state, whose
 *              value before rounding to fp32 is the unevaluated sum S_out + S_res
 *              (the state is carried with a compensation term through the sequence).
 *   z_res    : [G][D]    fp32 output, or NULL; NULL together with S_res.  Likewise.
 *              la_seq_bwd recovers the early states from the final carry; given these
 *              remainders it starts from the exact sum instead of its fp32 rounding,
 *              which matters for long sequences from a small initial carry.
 *   feature  : LA_FEATURE_NONE, or LA_FEATURE_ELU1: q and k hold raw inputs x and the
 *              op runs on phi(x) = elu(x) + 1 (x + 1 for x > 0, e^x otherwise),
 *              computed in fp32 as the inputs are loaded and rounded to bf16 (the
 *              positive feature map of the workloads, fused; section 1 needs q, k > 0).
 * Supported (block == 64, dt == LA_BF16):
 *   - D == 64: chunk == 128 and T a positive multiple of 128, T <= LA_SEQ_D64_MAX_T;
 *   - D == 128: chunk a positive multiple of 64, 1 <= T <= LA_SEQ_D128_MAX_T (the last
 *     chunk may be shorter than chunk, as a chain's last call may be).  Blocks of 64
 *     tokens start at multiples of 64 in both forms, so
 *     the chunk length does not change the arithmetic; a ragged end is computed as a
 *     masked block (the chained calls take it token by token: another summation order).
 * Anything else returns LA_ERR_UNSUPPORTED (chain la_chunk_fwd calls instead).  A
 * feature outside la_feature is LA_ERR_INVALID.
 */
la_status la_seq_fwd(const void *q, const void *k, const void *v,
                     const float *S_in, const float *z_in,
                     void *o, float *S_out, float *z_out, float *S_res, float *z_res,
                     int G, int T, int D, int chunk, int block, la_feature feature, la_dtype dt, void *stream);

/*
 * Backward over the same sequence for L = sum_t <dO_t, o_t> + <dS_out, S_out> +
 * dz_out . z_out: the reverse scan from the last chunk to the first, with the reverse
 * state passed on chip.
 *   q, k, v  : [G][T][D] dt, the forward's inputs.
 *   S_last   : [G][D][D] fp32, REQUIRED: the state after the last chunk, i.e. S_out of
 *              the la_seq_fwd call on these inputs.
 *   z_last   : [G][D]    fp32, REQUIRED: z_out of that call.
 *              The forward state before each chunk is recovered from (S_last, z_last)
 *              by subtracting the chunk's K^T V and K^T 1 (exact products of the
 *              inputs, summed in fp32), so no per-chunk carries are kept between the
 *              passes; the results differ from a chain of la_chunk_bwd calls only by
 *              that fp32 rounding (and, at D == 128, by the summation order of a
 *              ragged last block: a masked block here, token by token in the chunk
 *              call).  Passing anything but the forward's outputs gives the gradient
 *              at a different initial carry.
 *   S_res    : [G][D][D] fp32, or NULL: S_res of that la_seq_fwd call.
 *   z_res    : [G][D]    fp32, or NULL; NULL together with S_res.  With them the
 *              recovery starts from the exact final carry; without, from its fp32
 *              rounding, whose error reaches every earlier state (relative to the
 *              early states it grows with T: pass them for long sequences; the
 *              length limits hold with them).  At D == 128 the state is recovered
 *              without a compensation term (z with one), hence its shorter limit.
 *   dO       : [G][T][D] dt, gradient of o.
 *   dS_out   : [G][D][D] fp32 gradient of S_out, or NULL.
 *   dz_out   : [G][D]    fp32 gradient of z_out, or NULL; NULL together with dS_out.
 *   dq,dk,dv : [G][T][D] dt, outputs.
 *   dS_in    : [G][D][D] fp32 output, gradient of the carry before the first chunk.
 *   dz_in    : [G][D]    fp32 output.
 *   feature  : as in the forward call.  With LA_FEATURE_ELU1, dq and dk are the
 *              gradients with respect to the raw inputs: dq phi'(x_q), dk phi'(x_k)
 *              with phi'(x) = 1 for x > 0 and e^x otherwise (taken as min(1, phi)).
 * Supported: as la_seq_fwd.
 */
la_status la_seq_bwd(const void *q, const void *k, const void *v,
                     const float *S_last, const float *z_last, const float *S_res, const float *z_res,
                     const void *dO, const float *dS_out, const float *dz_out,
                     void *dq, void *dk, void *dv, float *dS_in, float *dz_in,
                     int G, int T, int D, int chunk, int block, la_feature feature, la_dtype dt, void *stream);

/*
 * Cross-entropy over a tied output head ("Fractus-1B training optimization", section 1,
 * Bottleneck #3: the 50257-token head; section 2, Opt 3: chunked, checkpointed cross-entropy):
 *     logit_iv = h_i . W_v,   lse_i = log sum_v exp(logit_iv),
 *     loss = (1/N) sum_i (lse_i - logit_{i,t_i}),
 * and for an upstream gradient g of the loss, with P_iv = (g/N) (softmax_iv - [v = t_i]),
 *     dh = P W,   dW = P^T h.
 *   h        : [N][d] bf16 hidden states (dt must be LA_BF16).
 *   W        : [V][d] bf16, the tied embedding (class v is row v).
 *   targets  : [N] int32 class of each token, each in [0, V) (not checked on the device: a
 *              target outside it gives a meaningless loss, nothing worse).
 *   loss     : fp32 scalar output (the mean over the N tokens).
 *   lse      : [N] fp32 output of the forward, input of the backward (its checkpoint: with
 *              it the backward forms each softmax from one recomputation of the logits).
 *   dloss    : fp32 scalar g on the device, or NULL for g = 1.
 *   dh       : [N][d] bf16 output;  dW : [V][d] fp32 output (overwritten).
 *   workspace: device scratch owned by the caller, 16-byte aligned, not read by the caller:
 *              at least la_ce_fwd_workspace_bytes(N, d, V) bytes for the forward (its
 *              per-tile partial sums: about 8 * N * V / 256 bytes, no logits) and
 *              la_ce_workspace_bytes(N, d, V, ce_chunk) for the backward, which is also
 *              enough for the forward, so one buffer of that size serves both calls (the
 *              backward's P of one chunk and the partial sums of dh).
 *   ce_chunk : tokens per backward chunk (1..N; anything else means N): the chunk's P,
 *              ce_chunk x V bf16, is the backward's only large transient.  The logits are
 *              never stored.
 * Supported: dt == LA_BF16, N >= 1, V >= 2, d a multiple of 128 up to 8192, V * d and
 * ceil(N / 128) * 128 * d below 2^30, and for the backward also
 * ceil(ce_chunk / 128) * 128 * ceil(V / 256) * 256 below 2^30 (32-bit byte offsets); the
 * workspace-size calls return 0 outside that set.  Each call launches several kernels
 * (la_time_next_launch brackets all of them).
 */
size_t la_ce_workspace_bytes(int N, int d, int V, int ce_chunk);
size_t la_ce_fwd_workspace_bytes(int N, int d, int V);
la_status la_ce_fwd(const void *h, const void *W, const int *targets, float *loss, float *lse,
                    void *workspace, size_t workspace_bytes, int N, int d, int V, la_dtype dt, void *stream);
la_status la_ce_bwd(const void *h, const void *W, const int *targets, const float *lse, const float *dloss,
                    void *dh, float *dW, void *workspace, size_t workspace_bytes,
                    int N, int d, int V, int ce_chunk, la_dtype dt, void *stream);

/*
 * la_ce_fwd for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same forward, same kernels and results,
 * but the workspace is the library's own static device array of LA_CE_NOALLOC_SCRATCH_BYTES,
 * one per GPU the library runs on, held until the process ends.  The caller passes only the
 * inputs and outputs (h, W, targets, loss, lse as for la_ce_fwd); nothing is allocated by the
 * call, the library or the caller.
 *   - Sizes whose forward workspace (la_ce_fwd_workspace_bytes) exceeds
 *     LA_CE_NOALLOC_SCRATCH_BYTES return LA_ERR_UNSUPPORTED (with V = 50257, up to 5248 tokens);
 *     otherwise the checks and statuses of la_ce_fwd apply.
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's contents (the
 *     forward overwrites all it reads, so nothing needs clearing).  Calls that overlap on one
 *     GPU (concurrent streams, or other host threads) race on it: serialise them.
 *   - The first call on a device looks up that device's copy of the array (hipGetSymbolAddress)
 *     and keeps its address; a failed lookup returns LA_ERR_LAUNCH.
 */
#define LA_CE_NOALLOC_SCRATCH_BYTES 8388608
la_status la_ce_fwd_noalloc(const void *h, const void *W, const int *targets, float *loss, float *lse,
                            int N, int d, int V, la_dtype dt, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *la_status_str(la_status s);

/* LA_ABI_VERSION of the built library. */
int la_abi_version(void);

/*
 * Measurement hook for benchmarks and profilers: the next la_chunk_fwd,
 * la_chunk_bwd, la_seq_fwd, la_seq_bwd, la_ce_fwd or la_ce_bwd call made by the
 * calling thread records start_event and stop_event (hipEvent_t, created by the
 * caller with timing enabled) on its kernel dispatches themselves, so
 * hipEventElapsedTime(start, stop) is the execution time with no marker packets in
 * between.  The attention entry points launch exactly one kernel; the
 * cross-entropy calls record start on their first dispatch and stop on their last.  The request is taken by that next call
 * whatever its status; (NULL, NULL) clears it.  Returns LA_ERR_INVALID if only
 * one event is given.  The events are not validated: they must be live events
 * of the device the next call runs on.
 */
la_status la_time_next_launch(void *start_event, void *stop_event);

/*
 * Measurement aid: the name of the kernel that la_chunk_fwd (backward = 0) or
 * la_chunk_bwd (backward = 1) launches for element type dt, chunk length C, head
 * dimension D, block and feature map, as it appears (demangled, template
 * arguments aside) in profiler output.  A static string; NULL when the
 * configuration is not supported.  Does not touch the device.
 */
const char *la_kernel_name(int backward, la_dtype dt, int C, int D, int block, la_feature feature);

/* The same for la_seq_fwd (backward = 0) and la_seq_bwd (backward = 1) at this chunk length. */
const char *la_seq_kernel_name(int backward, la_dtype dt, int chunk, int D, la_feature feature);

/*
 * Measurement aid: launch floors, kernels that do no arithmetic, for measuring what one launch
 * of a given size costs apart from any computation (nothing else in the library calls them).
 *   kind 0: an empty kernel of nwg workgroups; out must hold 512 * 4 bytes (never written),
 *           in is ignored;
 *   kind 1: nwg workgroups of 512 threads, each reading 65536 bytes of `in` (8 loads of 16 bytes
 *           per thread, all issued before the first is used) and writing 32768 bytes of `out`
 *           (non-temporal stores): at nwg = 160 the forward's bytes at the headline shape
 *           (160 groups, one 128-token chunk, D = 64, bf16: 10.5 MB read, 5.3 MB written);
 *   kind 2: the same with 81920 bytes read and 65536 written per workgroup: the backward's
 *           (13.2 MB read, 10.5 MB written at nwg = 160);
 *   kind 3, 4: kinds 1 and 2 in workgroups of 128 threads (a quarter of the bytes per
 *           workgroup): at nwg = 640 the same bytes as kinds 1 and 2 at nwg = 160.
 * in_bytes, out_bytes: the sizes of the device buffers, which must hold those counts times nwg
 * (LA_ERR_INVALID otherwise); 16-byte aligned; not overlapping.  la_time_next_launch applies.
 */
la_status la_floor_launch(int kind, int nwg, const void *in, size_t in_bytes, void *out, size_t out_bytes,
                          void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LA_CHUNK_H */
