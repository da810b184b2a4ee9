// Host side of the C ABI declared in include/la_chunk.h: argument validation,
// dispatch to the typed launchers, status strings, the launch-timing hook.
// Validation happens before any HIP call, so an invalid call touches neither
// the device nor the runtime.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/la_chunk.h"
#include "la_launch.h"

static_assert(LA_CE_NOALLOC_SCRATCH_BYTES == lachunk::CE_SCRATCH_BYTES, "the header states the scratch size");

namespace {

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};

bool mul_ok(size_t a, size_t b, size_t *out) {
    if (a != 0 && b > SIZE_MAX / a) return false;
    *out = a * b;
    return true;
}

bool overlap(const Span &a, const Span &b) {
    return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi;
}

Span span(const void *p, size_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{lo, p ? lo + bytes : lo};
}

bool aligned16(const void *p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int BK_TOKENS = 64;  // the block of the blocked form

struct Sizes {
    size_t tok, st, z;  // bytes of one token tensor, one state tensor, one normaliser
};

// Timing events for the next launch on this thread (la_time_next_launch); taken by that launch.
thread_local hipEvent_t pending_ev[2] = {nullptr, nullptr};

struct TakenEvents {
    hipEvent_t ev[2];
    TakenEvents() : ev{pending_ev[0], pending_ev[1]} { pending_ev[0] = pending_ev[1] = nullptr; }
};

la_status common_checks(int G, int C, int D, int block, la_dtype dt, Sizes *sz) {
    if (G < 1 || C < 1) return LA_ERR_INVALID;
    if (dt != LA_F32 && dt != LA_BF16) return LA_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return LA_ERR_UNSUPPORTED;
    if (block != 64 && block != 1) return LA_ERR_UNSUPPORTED;
    const size_t esz = dt == LA_F32 ? 4 : 2;
    size_t a, b;
    if (!mul_ok((size_t)G, (size_t)C, &a) || !mul_ok(a, (size_t)D, &b) || !mul_ok(b, esz, &sz->tok))
        return LA_ERR_INVALID;
    // the kernels address one group's chunk with 32-bit byte offsets (buffer resources),
    // with up to two windows of 128 tokens read past its end
    if ((size_t)C * D * esz + (size_t)256 * D * esz >= ((size_t)1 << 31)) return LA_ERR_UNSUPPORTED;
    if (!mul_ok((size_t)G, (size_t)D * D, &a) || !mul_ok(a, 4, &sz->st)) return LA_ERR_INVALID;
    sz->z = (size_t)G * D * 4;
    return LA_OK;
}

// Sequence entry points: the supported sets.  D = 64: bf16, 128-token chunks, whole chunks, T
// up to LA_SEQ_D64_MAX_T.  D = 128: bf16, chunks a multiple of the 64-token block (the last one
// may be ragged), T up to LA_SEQ_D128_MAX_T.  Both take the fused feature map.
la_status seq_checks(int G, int T, int D, int chunk, int block, la_dtype dt, la_feature feature, Sizes *sz) {
    if (G < 1 || T < 1 || chunk < 1) return LA_ERR_INVALID;
    if (feature != LA_FEATURE_NONE && feature != LA_FEATURE_ELU1) return LA_ERR_INVALID;
    la_status st = common_checks(G, chunk, D, block, dt, sz);
    if (st != LA_OK) return st;
    if (dt != LA_BF16 || block != BK_TOKENS) return LA_ERR_UNSUPPORTED;
    if (D == 64 && (chunk != 128 || T % chunk != 0 || T > LA_SEQ_D64_MAX_T)) return LA_ERR_UNSUPPORTED;
    if (D == 128 && (chunk % BK_TOKENS != 0 || T > LA_SEQ_D128_MAX_T)) return LA_ERR_UNSUPPORTED;
    size_t a, b;
    if (!mul_ok((size_t)G, (size_t)T, &a) || !mul_ok(a, (size_t)D * 2, &b)) return LA_ERR_INVALID;
    sz->tok = b;
    return LA_OK;
}

// Which kernel family a chunk call runs: the 128-token kernels (bf16, D = 64, C = 128, block 64);
// the D = 128 kernels (bf16, block 64: the sequence forward over a one-chunk sequence, and the
// backward that builds the carry after the chunk from the carry before it; forward chunks up to
// LA_SEQ_D128_MAX_T tokens); the per-token cumsum kernels (block 1; the fused feature map on any
// other shape; the fp32 backward at D = 128, whose blocked fp32 tiles exceed the LDS); or the
// general blocked kernels.
enum class Path { C128, D128, CUMSUM, GENERAL };
Path chunk_path(bool backward, la_dtype dt, int C, int D, int block, la_feature feature) {
    const bool c128 = dt == LA_BF16 && D == 64 && C == 128 && block == BK_TOKENS;
    if (c128) return Path::C128;
    if (dt == LA_BF16 && D == 128 && block == BK_TOKENS && (backward || C <= LA_SEQ_D128_MAX_T)) return Path::D128;
    if (block == 1 || feature == LA_FEATURE_ELU1 || (backward && dt == LA_F32 && D == 128)) return Path::CUMSUM;
    return Path::GENERAL;
}

// every output span against every input span and every other output span
la_status alias_checks(const Span *in, int nin, const Span *out, int nout) {
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlap(out[i], in[j])) return LA_ERR_ALIAS;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(out[i], out[j])) return LA_ERR_ALIAS;
    }
    return LA_OK;
}

}  // namespace

extern "C" {

la_status la_chunk_fwd(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                       void *o, float *S_out, float *z_out, int G, int C, int D, int block, la_feature feature,
                       la_dtype dt, void *stream) {
    const TakenEvents te;
    Sizes sz;
    if (feature != LA_FEATURE_NONE && feature != LA_FEATURE_ELU1) return LA_ERR_INVALID;
    la_status st = common_checks(G, C, D, block, dt, &sz);
    if (st != LA_OK) return st;
    if (!q || !k || !v || !o || !S_out || !z_out) return LA_ERR_INVALID;
    if ((S_in == nullptr) != (z_in == nullptr)) return LA_ERR_INVALID;
    const void *ptrs[] = {q, k, v, S_in, z_in, o, S_out, z_out};
    for (const void *p : ptrs)
        if (!aligned16(p)) return LA_ERR_ALIGN;
    const Span in[] = {span(q, sz.tok), span(k, sz.tok), span(v, sz.tok), span(S_in, sz.st), span(z_in, sz.z)};
    const Span out[] = {span(o, sz.tok), span(S_out, sz.st), span(z_out, sz.z)};
    st = alias_checks(in, 5, out, 3);
    if (st != LA_OK) return st;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool fm = feature == LA_FEATURE_ELU1;
    hipError_t e;
    const Path path = chunk_path(false, dt, C, D, block, feature);
    if (path == Path::C128)
        e = lachunk::launch_fwd_c128(q, k, v, S_in, z_in, o, S_out, z_out, G, fm, s, te.ev);
    else if (path == Path::D128)
        e = lachunk::launch_seq_fwd_d128(q, k, v, S_in, z_in, o, S_out, z_out, nullptr, nullptr, G, C, fm, s, te.ev);
    else if (path == Path::CUMSUM)
        e = dt == LA_BF16
                ? (D == 64 ? lachunk::launch_cumsum_fwd<__bf16, 64>(q, k, v, S_in, z_in, o, S_out, z_out, G, C, fm, s, te.ev)
                           : lachunk::launch_cumsum_fwd<__bf16, 128>(q, k, v, S_in, z_in, o, S_out, z_out, G, C, fm, s,
                                                                     te.ev))
                : (D == 64 ? lachunk::launch_cumsum_fwd<float, 64>(q, k, v, S_in, z_in, o, S_out, z_out, G, C, fm, s, te.ev)
                           : lachunk::launch_cumsum_fwd<float, 128>(q, k, v, S_in, z_in, o, S_out, z_out, G, C, fm, s,
                                                                    te.ev));
    else if (dt == LA_BF16)
        e = D == 64 ? lachunk::launch_fwd<__bf16, 64>(q, k, v, S_in, z_in, o, S_out, z_out, G, C, s, te.ev)
                    : lachunk::launch_fwd<__bf16, 128>(q, k, v, S_in, z_in, o, S_out, z_out, G, C, s, te.ev);
    else
        e = D == 64 ? lachunk::launch_fwd<float, 64>(q, k, v, S_in, z_in, o, S_out, z_out, G, C, s, te.ev)
                    : lachunk::launch_fwd<float, 128>(q, k, v, S_in, z_in, o, S_out, z_out, G, C, s, te.ev);
    return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_chunk_bwd(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                       const void *dO, const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv,
                       float *dS_in, float *dz_in, int G, int C, int D, int block, la_feature feature, la_dtype dt,
                       void *stream) {
    const TakenEvents te;
    Sizes sz;
    if (feature != LA_FEATURE_NONE && feature != LA_FEATURE_ELU1) return LA_ERR_INVALID;
    la_status st = common_checks(G, C, D, block, dt, &sz);
    if (st != LA_OK) return st;
    if (C > LA_BWD_MAX_C) return LA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !dO || !dq || !dk || !dv || !dS_in || !dz_in) return LA_ERR_INVALID;
    if ((S_in == nullptr) != (z_in == nullptr)) return LA_ERR_INVALID;
    if ((dS_out == nullptr) != (dz_out == nullptr)) return LA_ERR_INVALID;
    const void *ptrs[] = {q, k, v, S_in, z_in, dO, dS_out, dz_out, dq, dk, dv, dS_in, dz_in};
    for (const void *p : ptrs)
        if (!aligned16(p)) return LA_ERR_ALIGN;
    const Span in[] = {span(q, sz.tok),   span(k, sz.tok),      span(v, sz.tok),     span(S_in, sz.st),
                       span(z_in, sz.z), span(dO, sz.tok),     span(dS_out, sz.st), span(dz_out, sz.z)};
    const Span out[] = {span(dq, sz.tok), span(dk, sz.tok), span(dv, sz.tok), span(dS_in, sz.st),
                        span(dz_in, sz.z)};
    st = alias_checks(in, 8, out, 5);
    if (st != LA_OK) return st;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool fm = feature == LA_FEATURE_ELU1;
    hipError_t e;
    const Path path = chunk_path(true, dt, C, D, block, feature);
    if (path == Path::C128)
        e = lachunk::launch_bwd_c128(q, k, v, S_in, z_in, dO, dS_out, dz_out, dq, dk, dv, dS_in, dz_in, G, fm, s,
                                     te.ev);
    else if (path == Path::D128)
        e = lachunk::launch_bwd_d128(q, k, v, S_in, z_in, dO, dS_out, dz_out, dq, dk, dv, dS_in, dz_in, G, C, fm, s,
                                     te.ev);
    else if (path == Path::CUMSUM)
        e = dt == LA_BF16
                ? (D == 64 ? lachunk::launch_cumsum_bwd<__bf16, 64>(q, k, v, S_in, z_in, dO, dS_out, dz_out, dq, dk, dv,
                                                                    dS_in, dz_in, G, C, fm, s, te.ev)
                           : lachunk::launch_cumsum_bwd<__bf16, 128>(q, k, v, S_in, z_in, dO, dS_out, dz_out, dq, dk,
                                                                     dv, dS_in, dz_in, G, C, fm, s, te.ev))
                : (D == 64 ? lachunk::launch_cumsum_bwd<float, 64>(q, k, v, S_in, z_in, dO, dS_out, dz_out, dq, dk, dv,
                                                                   dS_in, dz_in, G, C, fm, s, te.ev)
                           : lachunk::launch_cumsum_bwd<float, 128>(q, k, v, S_in, z_in, dO, dS_out, dz_out, dq, dk, dv,
                                                                    dS_in, dz_in, G, C, fm, s, te.ev));
    else if (dt == LA_BF16)
        e = D == 64 ? lachunk::launch_bwd<__bf16, 64>(q, k, v, S_in, z_in, dO, dS_out, dz_out, dq, dk, dv, dS_in,
                                                     dz_in, G, C, s, te.ev)
                    : lachunk::launch_bwd<__bf16, 128>(q, k, v, S_in, z_in, dO, dS_out, dz_out, dq, dk, dv, dS_in,
                                                      dz_in, G, C, s, te.ev);
    else
        e = lachunk::launch_bwd<float, 64>(q, k, v, S_in, z_in, dO, dS_out, dz_out, dq, dk, dv, dS_in, dz_in, G, C,
                                           s, te.ev);
    return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_seq_fwd(const void *q, const void *k, const void *v, const float *S_in, const float *z_in, void *o,
                     float *S_out, float *z_out, float *S_res, float *z_res, int G, int T, int D, int chunk,
                     int block, la_feature feature, la_dtype dt, void *stream) {
    const TakenEvents te;
    Sizes sz;
    la_status st = seq_checks(G, T, D, chunk, block, dt, feature, &sz);
    if (st != LA_OK) return st;
    if (!q || !k || !v || !o || !S_out || !z_out) return LA_ERR_INVALID;
    if ((S_in == nullptr) != (z_in == nullptr) || (S_res == nullptr) != (z_res == nullptr)) return LA_ERR_INVALID;
    const void *ptrs[] = {q, k, v, S_in, z_in, o, S_out, z_out, S_res, z_res};
    for (const void *p : ptrs)
        if (!aligned16(p)) return LA_ERR_ALIGN;
    const Span in[] = {span(q, sz.tok), span(k, sz.tok), span(v, sz.tok), span(S_in, sz.st), span(z_in, sz.z)};
    const Span out[] = {span(o, sz.tok), span(S_out, sz.st), span(z_out, sz.z), span(S_res, sz.st),
                        span(z_res, sz.z)};
    st = alias_checks(in, 5, out, 5);
    if (st != LA_OK) return st;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // D = 128: one workgroup per group walks the whole sequence (la_seq_fwd_d128_kernel)
    const hipError_t e =
        D == 128 ? lachunk::launch_seq_fwd_d128(q, k, v, S_in, z_in, o, S_out, z_out, S_res, z_res, G, T,
                                                feature == LA_FEATURE_ELU1, s, te.ev)
                 : lachunk::launch_seq_fwd_c128(q, k, v, S_in, z_in, o, S_out, z_out, S_res, z_res, G, T / chunk,
                                                feature == LA_FEATURE_ELU1, s, te.ev);
    return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_seq_bwd(const void *q, const void *k, const void *v, const float *S_last, const float *z_last,
                     const float *S_res, const float *z_res, const void *dO, const float *dS_out,
                     const float *dz_out, void *dq, void *dk, void *dv, float *dS_in, float *dz_in, int G, int T,
                     int D, int chunk, int block, la_feature feature, la_dtype dt, void *stream) {
    const TakenEvents te;
    Sizes sz;
    la_status st = seq_checks(G, T, D, chunk, block, dt, feature, &sz);
    if (st != LA_OK) return st;
    if (!q || !k || !v || !S_last || !z_last || !dO || !dq || !dk || !dv || !dS_in || !dz_in) return LA_ERR_INVALID;
    if ((dS_out == nullptr) != (dz_out == nullptr) || (S_res == nullptr) != (z_res == nullptr))
        return LA_ERR_INVALID;
    const void *ptrs[] = {q, k, v, S_last, z_last, S_res, z_res, dO, dS_out, dz_out, dq, dk, dv, dS_in, dz_in};
    for (const void *p : ptrs)
        if (!aligned16(p)) return LA_ERR_ALIGN;
    const Span in[] = {span(q, sz.tok),     span(k, sz.tok),     span(v, sz.tok),    span(S_last, sz.st),
                       span(z_last, sz.z),  span(S_res, sz.st),  span(z_res, sz.z),  span(dO, sz.tok),
                       span(dS_out, sz.st), span(dz_out, sz.z)};
    const Span out[] = {span(dq, sz.tok), span(dk, sz.tok), span(dv, sz.tok), span(dS_in, sz.st),
                        span(dz_in, sz.z)};
    st = alias_checks(in, 10, out, 5);
    if (st != LA_OK) return st;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const hipError_t e =
        D == 128 ? lachunk::launch_seq_bwd_d128(q, k, v, S_last, z_last, S_res, z_res, dO, dS_out, dz_out, dq, dk,
                                                dv, dS_in, dz_in, G, T, feature == LA_FEATURE_ELU1, s, te.ev)
                 : lachunk::launch_seq_bwd_c128(q, k, v, S_last, z_last, S_res, z_res, dO, dS_out, dz_out, dq, dk,
                                                dv, dS_in, dz_in, G, T / chunk, feature == LA_FEATURE_ELU1, s, te.ev);
    return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

// Cross-entropy: the shapes the forward supports (its kernels address h and W with 32-bit byte
// offsets; the partials are indexed in 64 bits).  The forward's workspace is s->fwd_bytes.
static la_status ce_fwd_checks(int N, int d, int V, la_dtype dt, lachunk::CeShape *s) {
    if (N < 1 || d < 1 || V < 2) return LA_ERR_INVALID;
    if (dt != LA_BF16 || d % 128 != 0 || d > 8192) return LA_ERR_UNSUPPORTED;
    *s = lachunk::ce_shape(N, d, V, N);
    if ((size_t)V * d >= ((size_t)1 << 30) || (size_t)s->Npad * d >= ((size_t)1 << 30)) return LA_ERR_UNSUPPORTED;
    return LA_OK;
}

// The backward's, at this chunk: P of one chunk is also addressed with 32-bit byte offsets.  Its
// workspace is s->bwd_bytes.
static la_status ce_bwd_checks(int N, int d, int V, int ce_chunk, la_dtype dt, lachunk::CeShape *s) {
    la_status st = ce_fwd_checks(N, d, V, dt, s);
    if (st != LA_OK) return st;
    *s = lachunk::ce_shape(N, d, V, ce_chunk);
    if ((size_t)s->chunk_pad * s->Vpad >= ((size_t)1 << 30)) return LA_ERR_UNSUPPORTED;
    return LA_OK;
}

size_t la_ce_workspace_bytes(int N, int d, int V, int ce_chunk) {
    lachunk::CeShape s;
    return ce_bwd_checks(N, d, V, ce_chunk, LA_BF16, &s) == LA_OK ? s.ws_bytes : 0;
}

size_t la_ce_fwd_workspace_bytes(int N, int d, int V) {
    lachunk::CeShape s;
    return ce_fwd_checks(N, d, V, LA_BF16, &s) == LA_OK ? s.fwd_bytes : 0;
}

la_status la_ce_fwd(const void *h, const void *W, const int *targets, float *loss, float *lse, void *workspace,
                    size_t workspace_bytes, int N, int d, int V, la_dtype dt, void *stream) {
    const TakenEvents te;
    lachunk::CeShape s;
    la_status st = ce_fwd_checks(N, d, V, dt, &s);
    if (st != LA_OK) return st;
    if (!h || !W || !targets || !loss || !lse || !workspace) return LA_ERR_INVALID;
    if (workspace_bytes < s.fwd_bytes) return LA_ERR_INVALID;
    const void *ptrs[] = {h, W, targets, loss, lse, workspace};
    for (const void *p : ptrs)
        if (!aligned16(p)) return LA_ERR_ALIGN;
    const Span in[] = {span(h, (size_t)N * d * 2), span(W, (size_t)V * d * 2), span(targets, (size_t)N * 4)};
    const Span out[] = {span(loss, 4), span(lse, (size_t)N * 4), span(workspace, workspace_bytes)};
    st = alias_checks(in, 3, out, 3);
    if (st != LA_OK) return st;
    const hipError_t e = lachunk::launch_ce_fwd(h, W, targets, loss, lse, workspace, N, d, V,
                                                reinterpret_cast<hipStream_t>(stream), te.ev);
    return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_ce_fwd_noalloc(const void *h, const void *W, const int *targets, float *loss, float *lse, int N, int d,
                            int V, la_dtype dt, void *stream) {
    const TakenEvents te;
    lachunk::CeShape s;
    la_status st = ce_fwd_checks(N, d, V, dt, &s);
    if (st != LA_OK) return st;
    if (s.fwd_bytes > LA_CE_NOALLOC_SCRATCH_BYTES) return LA_ERR_UNSUPPORTED;
    if (!h || !W || !targets || !loss || !lse) return LA_ERR_INVALID;
    const void *ptrs[] = {h, W, targets, loss, lse};
    for (const void *p : ptrs)
        if (!aligned16(p)) return LA_ERR_ALIGN;
    const Span in[] = {span(h, (size_t)N * d * 2), span(W, (size_t)V * d * 2), span(targets, (size_t)N * 4)};
    const Span out[] = {span(loss, 4), span(lse, (size_t)N * 4)};
    st = alias_checks(in, 3, out, 2);
    if (st != LA_OK) return st;
    const hipError_t e = lachunk::launch_ce_fwd_noalloc(h, W, targets, loss, lse, N, d, V,
                                                        reinterpret_cast<hipStream_t>(stream), te.ev);
    return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_ce_bwd(const void *h, const void *W, const int *targets, const float *lse, const float *dloss, void *dh,
                    float *dW, void *workspace, size_t workspace_bytes, int N, int d, int V, int ce_chunk,
                    la_dtype dt, void *stream) {
    const TakenEvents te;
    lachunk::CeShape s;
    la_status st = ce_bwd_checks(N, d, V, ce_chunk, dt, &s);
    if (st != LA_OK) return st;
    if (!h || !W || !targets || !lse || !dh || !dW || !workspace) return LA_ERR_INVALID;
    if (workspace_bytes < s.bwd_bytes) return LA_ERR_INVALID;
    const void *ptrs[] = {h, W, targets, lse, dloss, dh, dW, workspace};
    for (const void *p : ptrs)
        if (!aligned16(p)) return LA_ERR_ALIGN;
    const Span in[] = {span(h, (size_t)N * d * 2), span(W, (size_t)V * d * 2), span(targets, (size_t)N * 4),
                       span(lse, (size_t)N * 4), span(dloss, 4)};
    const Span out[] = {span(dh, (size_t)N * d * 2), span(dW, (size_t)V * d * 4), span(workspace, workspace_bytes)};
    st = alias_checks(in, 5, out, 3);
    if (st != LA_OK) return st;
    const hipError_t e = lachunk::launch_ce_bwd(h, W, targets, lse, dloss, dh, dW, workspace, N, d, V, s.chunk,
                                                reinterpret_cast<hipStream_t>(stream), te.ev);
    return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

const char *la_status_str(la_status s) {
    switch (s) {
        case LA_OK: return "ok";
        case LA_ERR_INVALID: return "invalid argument (null pointer, non-positive size, half-given carry or overflow)";
        case LA_ERR_UNSUPPORTED: return "unsupported configuration (D, block, dtype or chunk length)";
        case LA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case LA_ERR_ALIAS: return "an output buffer overlaps an input or another output";
        case LA_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

int la_abi_version(void) { return LA_ABI_VERSION; }

const char *la_kernel_name(int backward, la_dtype dt, int C, int D, int block, la_feature feature) {
    if ((dt != LA_F32 && dt != LA_BF16) || (D != 64 && D != 128) || C < 1 || (block != 64 && block != 1)) return nullptr;
    if (feature != LA_FEATURE_NONE && feature != LA_FEATURE_ELU1) return nullptr;
    if (backward && C > LA_BWD_MAX_C) return nullptr;
    const bool fm = feature == LA_FEATURE_ELU1;
    switch (chunk_path(backward != 0, dt, C, D, block, feature)) {
        case Path::C128:
            if (backward) return fm ? "la_bwd_c128w16_elu1_kernel" : "la_bwd_c128w16_kernel";
            return fm ? "la_fwd_c128_elu1_kernel" : "la_fwd_c128_kernel";
        case Path::D128:
            if (backward) return fm ? "la_bwd_d128_elu1_kernel" : "la_bwd_d128_kernel";
            return fm ? "la_seq_fwd_d128_elu1_kernel" : "la_seq_fwd_d128_kernel";
        case Path::CUMSUM: return backward ? "la_cumsum_bwd_kernel" : "la_cumsum_fwd_kernel";
        case Path::GENERAL: break;
    }
    return backward ? "la_bwd_kernel" : "la_fwd_kernel";
}

const char *la_seq_kernel_name(int backward, la_dtype dt, int chunk, int D, la_feature feature) {
    if (feature != LA_FEATURE_NONE && feature != LA_FEATURE_ELU1) return nullptr;
    const bool fm = feature == LA_FEATURE_ELU1;
    if (dt == LA_BF16 && D == 128 && chunk >= BK_TOKENS && chunk % BK_TOKENS == 0) {
        if (fm) return backward ? "la_seq_bwd_d128_elu1_kernel" : "la_seq_fwd_d128_elu1_kernel";
        return backward ? "la_seq_bwd_d128_kernel" : "la_seq_fwd_d128_kernel";
    }
    if (dt != LA_BF16 || D != 64 || chunk != 128) return nullptr;
    if (fm) return backward ? "la_seq_bwd_c128w16_elu1_kernel" : "la_seq_fwd_c128_elu1_kernel";
    return backward ? "la_seq_bwd_c128w16_kernel" : "la_seq_fwd_c128_kernel";
}

la_status la_floor_launch(int kind, int nwg, const void *in, size_t in_bytes, void *out, size_t out_bytes,
                          void *stream) {
    const TakenEvents te;
    if (kind < 0 || kind >= lachunk::FLOOR_KINDS || nwg < 1) return LA_ERR_INVALID;
    int nin, nout, nt;
    lachunk::floor_shape(kind, &nin, &nout, &nt);
    const size_t per_in = (size_t)nin * nt * 16, per_out = (size_t)nout * nt * 16;
    // the empty kernel's only pointer is never written, but must be a device buffer of 4 bytes per thread
    const size_t need_out = kind == 0 ? (size_t)lachunk::FLOOR_THREADS * 4 : (size_t)nwg * per_out;
    if (!out || out_bytes < need_out || (kind != 0 && (!in || in_bytes < (size_t)nwg * per_in))) return LA_ERR_INVALID;
    if (!aligned16(in) || !aligned16(out)) return LA_ERR_ALIGN;
    if (kind != 0 && overlap(span(in, (size_t)nwg * per_in), span(out, need_out))) return LA_ERR_ALIAS;
    const hipError_t e = lachunk::launch_floor(kind, nwg, in, out, reinterpret_cast<hipStream_t>(stream), te.ev);
    return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_time_next_launch(void *start_event, void *stop_event) {
    if ((start_event == nullptr) != (stop_event == nullptr)) return LA_ERR_INVALID;
    pending_ev[0] = reinterpret_cast<hipEvent_t>(start_event);
    pending_ev[1] = reinterpret_cast<hipEvent_t>(stop_event);
    return LA_OK;
}

}  // extern "C"
