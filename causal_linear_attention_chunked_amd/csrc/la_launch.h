// Typed launchers, one per supported (element type, head dim) pair.  Each
// enqueues its kernel on `stream` and returns the launch status.  `ev` holds
// two hipEvent_t (start, stop) recorded on the dispatch itself, or nulls.
#pragma once
#include <hip/hip_runtime.h>

namespace lachunk {

template <typename T, int D>
hipError_t launch_fwd(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                      void *o, float *S_out, float *z_out, int G, int C, hipStream_t stream,
                      const hipEvent_t ev[2]);

template <typename T, int D>
hipError_t launch_bwd(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                      const void *dO, const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv,
                      float *dS_in, float *dz_in, int G, int C, hipStream_t stream,
                      const hipEvent_t ev[2]);

// bf16, D = 64, exactly two blocks (C = 128): both blocks of the chunk worked on side by side;
// elu1: q and k are raw inputs and the feature map elu(x) + 1 is applied inside.
hipError_t launch_fwd_c128(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                           void *o, float *S_out, float *z_out, int G, bool elu1, hipStream_t stream,
                           const hipEvent_t ev[2]);
hipError_t launch_bwd_c128(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                           const void *dO, const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv,
                           float *dS_in, float *dz_in, int G, bool elu1, hipStream_t stream, const hipEvent_t ev[2]);

// The cumsum form: the per-token recurrence over one chunk of any length (backward: C up to
// LA_BWD_MAX_C), fp32 arithmetic, any supported element type and D; elu1 as above.
template <typename T, int D>
hipError_t launch_cumsum_fwd(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                             void *o, float *S_out, float *z_out, int G, int C, bool elu1, hipStream_t stream,
                             const hipEvent_t ev[2]);
template <typename T, int D>
hipError_t launch_cumsum_bwd(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                             const void *dO, const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv,
                             float *dS_in, float *dz_in, int G, int C, bool elu1, hipStream_t stream,
                             const hipEvent_t ev[2]);

// The same kernels walking a group's nchunk consecutive 128-token chunks, carry on chip
// (backward: S_last / z_last is the state after the last chunk); elu1: q and k are raw inputs
// and the feature map elu(x) + 1 is applied inside.  The final carry is exact as the unevaluated
// sum (S_out + S_res, z_out + z_res): the forward writes the remainders where the pointers are
// not null, the backward starts from them (null: zero).
hipError_t launch_seq_fwd_c128(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                               void *o, float *S_out, float *z_out, float *S_res, float *z_res, int G, int nchunk,
                               bool elu1, hipStream_t stream, const hipEvent_t ev[2]);
hipError_t launch_seq_bwd_c128(const void *q, const void *k, const void *v, const float *S_last,
                               const float *z_last, const float *S_res, const float *z_res, const void *dO,
                               const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv, float *dS_in,
                               float *dz_in, int G, int nchunk, bool elu1, hipStream_t stream,
                               const hipEvent_t ev[2]);

// bf16, D = 128: the forward over a whole sequence of T tokens per group (any T >= 1; a ragged
// end is a masked block), S and z carried with compensation, remainders out as above.
hipError_t launch_seq_fwd_d128(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                               void *o, float *S_out, float *z_out, float *S_res, float *z_res, int G, int T,
                               bool elu1, hipStream_t stream, const hipEvent_t ev[2]);

// bf16, D = 128: the backward over a whole sequence of T tokens per group (any T >= 1, the last
// 64-token block possibly ragged), last block first, from the carry after the last token.
hipError_t launch_seq_bwd_d128(const void *q, const void *k, const void *v, const float *S_last,
                               const float *z_last, const float *S_res, const float *z_res, const void *dO,
                               const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv, float *dS_in,
                               float *dz_in, int G, int T, bool elu1, hipStream_t stream, const hipEvent_t ev[2]);

// bf16, D = 128: the backward over one chunk of C tokens (C >= 1, the last 64-token block possibly
// ragged) from the carry before it: the carry after the chunk is built first, then the reverse walk
// of launch_seq_bwd_d128.
hipError_t launch_bwd_d128(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                           const void *dO, const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv,
                           float *dS_in, float *dz_in, int G, int C, bool elu1, hipStream_t stream,
                           const hipEvent_t ev[2]);

// Cross-entropy over a tied head (bf16 h, W; fp32 loss, lse, dW; bf16 dh).  The GEMM tiles
// (CE_MT class rows x CE_NT tokens, CE_CK k per stage) and the shape of the workspace: padded
// sizes, the backward's chunking and the split of dh over the vocabulary.  Host arithmetic
// only (the argument checks use it too).
constexpr int CE_MT = 256, CE_NT = 128, CE_CK = 64;
struct CeShape {
    int Npad, Vpad, nvt, chunk, chunk_pad, kper, nsplit;
    size_t fwd_bytes, p_bytes, bwd_bytes, ws_bytes;
};
inline CeShape ce_shape(int N, int d, int V, int ce_chunk) {
    CeShape s;
    s.Npad = (N + CE_NT - 1) / CE_NT * CE_NT;
    s.Vpad = (V + CE_MT - 1) / CE_MT * CE_MT;  // whole class tiles of the forward and of P
    s.nvt = s.Vpad / CE_MT;
    s.chunk = ce_chunk < 1 || ce_chunk > N ? N : ce_chunk;
    s.chunk_pad = (s.chunk + CE_NT - 1) / CE_NT * CE_NT;
    // dh split over the vocabulary: at most one workgroup per compute unit (256), whole k-steps
    // per split
    const int tiles = (d + CE_MT - 1) / CE_MT * (s.chunk_pad / CE_NT);
    int nsplit = tiles >= 256 ? 1 : 256 / tiles;
    if (nsplit > s.Vpad / CE_CK) nsplit = s.Vpad / CE_CK;
    s.kper = ((s.Vpad + nsplit - 1) / nsplit + CE_CK - 1) / CE_CK * CE_CK;
    s.nsplit = (s.Vpad + s.kper - 1) / s.kper;
    s.fwd_bytes = (size_t)s.nvt * s.Npad * 8 + (size_t)s.Npad * 8;  // partials, target logits, nll
    s.p_bytes = (size_t)s.chunk_pad * s.Vpad * 2;
    s.bwd_bytes = s.p_bytes + (size_t)s.nsplit * s.chunk_pad * d * 4;
    s.ws_bytes = s.fwd_bytes > s.bwd_bytes ? s.fwd_bytes : s.bwd_bytes;
    return s;
}
hipError_t launch_ce_fwd(const void *h, const void *W, const int *targets, float *loss, float *lse, void *ws, int N,
                         int d, int V, hipStream_t stream, const hipEvent_t ev[2]);
// The same forward with the library's own per-device scratch array (CE_SCRATCH_BYTES, a static
// device array) as its workspace: nothing is allocated by the library or the caller.
constexpr size_t CE_SCRATCH_BYTES = (size_t)8 << 20;
hipError_t launch_ce_fwd_noalloc(const void *h, const void *W, const int *targets, float *loss, float *lse, int N,
                                 int d, int V, hipStream_t stream, const hipEvent_t ev[2]);
hipError_t launch_ce_bwd(const void *h, const void *W, const int *targets, const float *lse, const float *dloss,
                         void *dh, float *dW, void *ws, int N, int d, int V, int ce_chunk, hipStream_t stream,
                         const hipEvent_t ev[2]);

// Launch floors (measurement aid): kind 0 an empty kernel; kinds 1 and 2 streaming kernels whose
// workgroups of FLOOR_THREADS threads each issue nin 16-byte loads per thread up front and then
// nout stores: the forward's and the backward's bytes per group at the headline shape; kinds 3
// and 4 the same per thread in workgroups of FLOOR_SMALL_THREADS threads (the same bytes over
// four times the workgroups).
constexpr int FLOOR_THREADS = 512, FLOOR_SMALL_THREADS = 128;
constexpr int FLOOR_FWD_NIN = 8, FLOOR_FWD_NOUT = 4, FLOOR_BWD_NIN = 10, FLOOR_BWD_NOUT = 8;
constexpr int FLOOR_KINDS = 5;
inline void floor_shape(int kind, int *nin, int *nout, int *nthreads) {
    const bool fwd = kind == 1 || kind == 3, bwd = kind == 2 || kind == 4;
    *nin = fwd ? FLOOR_FWD_NIN : bwd ? FLOOR_BWD_NIN : 0;
    *nout = fwd ? FLOOR_FWD_NOUT : bwd ? FLOOR_BWD_NOUT : 0;
    *nthreads = kind >= 3 ? FLOOR_SMALL_THREADS : FLOOR_THREADS;
}
hipError_t launch_floor(int kind, int nwg, const void *in, void *out, hipStream_t stream, const hipEvent_t ev[2]);

}  // namespace lachunk
