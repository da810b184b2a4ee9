// The cumsum form of causal linear attention: the exact per-token recurrence, token after token,
// with no blocking ("Fractus-1B training optimization", section 1, Bottleneck #1: the state as a
// running sum of k v^T read after the update that includes the token; section 2, Opt 1 and
// Opt 2 name it among the selectable attention forms and as the exact fallback of the chunked
// one).  The backward is the reverse scan of the same section (the gradient of a prefix sum is a
// suffix sum):
//   forward, t = 1..C:  S += k_t v_t^T,  z += k_t,  den_t = q_t . z,  o_t = S^T q_t / den_t
//   backward, pass 1 in order:   the same, then dn_t = dO_t / den_t, dden_t = -(dO_t . o_t) / den_t,
//                                dq_t = S dn_t + dden_t z
//   backward, pass 2 in reverse: Sh += q_t dn_t^T, zh += dden_t q_t, dk_t = Sh v_t + zh, dv_t = Sh^T k_t
//   from Sh = dS_out, zh = dz_out; dS_in = Sh, dz_in = zh at the end.
// Everything is fp32 arithmetic on the stored inputs (bf16 or fp32); no MFMA: each token is a
// rank-one update and two matrix-vector products, vector work.
//
// One workgroup per group, D / 16 waves.  Wave w owns value columns 16w .. 16w + 15; in a wave,
// lane (r, g) = (lane % 16, lane / 16) owns column c = 16w + r and key features
// p = g NP .. g NP + NP - 1 (NP = D / 4) of the state (layout A: S[p][c], with z[p]); column sums
// over p are sums over the four lane groups (gsum).  The backward also keeps the state as rows
// (layout B: lane owns row p = 16w + r and columns g NP ..; S[p][c], with z[p]) for the products
// that sum over c.  Tokens are staged 32 at a time through LDS (each thread's share of the next
// batch is loaded into registers while the current batch is worked on) and outputs leave
// through an LDS tile, one coalesced store per batch.
#include "la_tile.h"
#include "la_launch.h"
#include "../../include/la_chunk.h"
#include <hip/hip_ext.h>

namespace lachunk {

namespace {

template <typename T, int D>
struct Cumsum {
    static constexpr int NW = D / 16;            // waves
    static constexpr int NTH = 64 * NW;          // threads (4 D: the kernels' launch bounds)
    static constexpr int NP = D / 4;             // key features per lane group
    static constexpr int BT = 32;                // tokens per staged batch
    static constexpr int TILE = BT * D * (int)sizeof(T);  // bytes of one staged tensor
    static constexpr int VB = TILE / NTH;        // bytes per thread per tensor (16 or 32)
    static constexpr int NV = VB / 16;           // 16-byte loads per thread per tensor
    static_assert(VB % 16 == 0 && NV >= 1, "whole 16-byte loads");
};

typedef int int4v __attribute__((ext_vector_type(4)));

// A thread's share of one batch of one tensor: NV 16-byte pieces at byte offset tid * VB + 16 i
// of the batch (the batch is BT consecutive rows, one contiguous span); reads past the range
// (past the chunk) give zeros.
template <int NV>
struct Share {
    int4v x[NV];
    __device__ __forceinline__ void load(const GRes &g, uint32_t batch_off, int tid) {
#pragma unroll
        for (int i = 0; i < NV; ++i) x[i] = gload<int4v>(g, batch_off + (uint32_t)(tid * NV + i) * 16);
    }
    __device__ __forceinline__ void store(char *tile, int tid) const {
#pragma unroll
        for (int i = 0; i < NV; ++i) *reinterpret_cast<int4v *>(tile + (tid * NV + i) * 16) = x[i];
    }
    // The same through the positive feature map phi(x) = elu(x) + 1 (raw q, k in), computed in
    // fp32 and rounded to the element type T.
    template <typename T>
    __device__ __forceinline__ void store_mapped(char *tile, int tid) const {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int4v y;
            if constexpr (sizeof(T) == 2) {
                y = __builtin_bit_cast(int4v, elu1_8(__builtin_bit_cast(bf16x8, x[i])));
            } else {
                const floatx4 f = __builtin_bit_cast(floatx4, x[i]);
                y = __builtin_bit_cast(int4v, floatx4{elu1_f(f[0]), elu1_f(f[1]), elu1_f(f[2]), elu1_f(f[3])});
            }
            *reinterpret_cast<int4v *>(tile + (tid * NV + i) * 16) = y;
        }
    }
};

// Four consecutive elements of an LDS row as fp32 (read where they are used, four at a time, so
// that only a few of a row's values are live at once).
template <typename T>
__device__ __forceinline__ floatx4 quad(const T *row) {
    const Vec4<T> x = *reinterpret_cast<const Vec4<T> *>(row);
    return floatx4{tof(x[0]), tof(x[1]), tof(x[2]), tof(x[3])};
}

// Writes the first n rows of an output tile (row pitch D) to global rows row0.., coalesced in
// 16-byte pieces; a ragged batch stores whole pieces of its valid rows only.
template <typename T, int D, int NTH>
__device__ __forceinline__ void flush_tile(const char *tile, T *dst_rows, int n, int tid) {
    constexpr int PIECES_PER_ROW = D * (int)sizeof(T) / 16;
    const int total = n * PIECES_PER_ROW;
    for (int i = tid; i < total; i += NTH)
        reinterpret_cast<int4v *>(dst_rows)[i] = reinterpret_cast<const int4v *>(tile)[i];
}

}  // namespace

template <typename T, int D, bool FM>
__global__ __launch_bounds__(4 * D, 1) void la_cumsum_fwd_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ S_in,
    const float *__restrict__ z_in, T *__restrict__ o, float *__restrict__ S_out, float *__restrict__ z_out, int C) {
    using K = Cumsum<T, D>;
    constexpr int NP = K::NP, BT = K::BT;
    __shared__ __attribute__((aligned(16))) char smem[4 * K::TILE];
    char *const tq = smem, *const tk = smem + K::TILE, *const tv = smem + 2 * K::TILE, *const to = smem + 3 * K::TILE;
    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = 16 * w + r, p0 = g * NP;
    const size_t grp = blockIdx.x, tok0 = grp * (size_t)C;
    const uint32_t bytes = (uint32_t)C * D * sizeof(T);
    const GRes qr(q + tok0 * D, bytes), kr(k + tok0 * D, bytes), vr(v + tok0 * D, bytes);
    const float *dummy = S_out;  // a valid base for an empty range (an absent carry reads zeros)
    const GRes sres(S_in ? (const void *)(S_in + grp * D * D) : dummy, S_in ? D * D * 4 : 0);
    const GRes zres(z_in ? (const void *)(z_in + grp * D) : dummy, z_in ? D * 4 : 0);

    float SA[NP], zA[NP];
#pragma unroll
    for (int s = 0; s < NP; ++s) {
        SA[s] = gload<float>(sres, ((p0 + s) * D + c) * 4);
        zA[s] = gload<float>(zres, (p0 + s) * 4);
    }
    Share<K::NV> sq, sk, sv;
    sq.load(qr, 0, tid);
    sk.load(kr, 0, tid);
    sv.load(vr, 0, tid);
    const int nbatch = (C + BT - 1) / BT;
    for (int b = 0; b < nbatch; ++b) {
        __syncthreads();  // the previous batch's tiles are read and its outputs stored
        if constexpr (FM) {  // fused feature map: raw q, k mapped as they are staged
            sq.template store_mapped<T>(tq, tid);
            sk.template store_mapped<T>(tk, tid);
        } else {
            sq.store(tq, tid);
            sk.store(tk, tid);
        }
        sv.store(tv, tid);
        __syncthreads();
        const uint32_t next = (uint32_t)(b + 1) * K::TILE;  // past the chunk: reads give zero
        sq.load(qr, next, tid);
        sk.load(kr, next, tid);
        sv.load(vr, next, tid);
        const int n = C - b * BT < BT ? C - b * BT : BT;
        for (int t = 0; t < n; ++t) {
            const T *qt = reinterpret_cast<const T *>(tq) + t * D, *kt = reinterpret_cast<const T *>(tk) + t * D;
            const float vc = tof(reinterpret_cast<const T *>(tv)[t * D + c]);
            float d[2] = {0.f, 0.f}, nn[2] = {0.f, 0.f};
#pragma unroll
            for (int s0 = 0; s0 < NP; s0 += 4) {
                const floatx4 kp = quad(kt + p0 + s0), qp = quad(qt + p0 + s0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = s0 + e;
                    zA[s] += kp[e];
                    SA[s] = __builtin_fmaf(kp[e], vc, SA[s]);
                    d[e & 1] = __builtin_fmaf(qp[e], zA[s], d[e & 1]);
                    nn[e & 1] = __builtin_fmaf(qp[e], SA[s], nn[e & 1]);
                }
            }
            const float den = gsum(d[0] + d[1]), num = gsum(nn[0] + nn[1]);
            if (g == 0) reinterpret_cast<T *>(to)[t * D + c] = fromf<T>(num / den);
        }
        __syncthreads();  // the batch's outputs are in the tile
        flush_tile<T, D, K::NTH>(to, o + (tok0 + (size_t)b * BT) * D, n, tid);
    }
#pragma unroll
    for (int s = 0; s < NP; ++s) S_out[grp * D * D + (size_t)(p0 + s) * D + c] = SA[s];
    if (w == 0 && r == 0) {
#pragma unroll
        for (int s = 0; s < NP; ++s) z_out[grp * D + p0 + s] = zA[s];
    }
}

template <typename T, int D, bool FM>
__global__ __launch_bounds__(4 * D, 1) void la_cumsum_bwd_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ S_in,
    const float *__restrict__ z_in, const T *__restrict__ dO, const float *__restrict__ dS_out,
    const float *__restrict__ dz_out, T *__restrict__ dq, T *__restrict__ dk, T *__restrict__ dv,
    float *__restrict__ dS_in, float *__restrict__ dz_in, int C) {
    using K = Cumsum<T, D>;
    constexpr int NP = K::NP, BT = K::BT, NW = K::NW;
    constexpr int OFF_DEN = 6 * K::TILE, OFF_DDEN = OFF_DEN + LA_BWD_MAX_C * 4, OFF_PART = OFF_DDEN + LA_BWD_MAX_C * 4;
    __shared__ __attribute__((aligned(16))) char smem[OFF_PART + 2 * NW * 4];
    char *const tq = smem, *const tk = smem + K::TILE, *const tv = smem + 2 * K::TILE, *const tg = smem + 3 * K::TILE;
    char *const to1 = smem + 4 * K::TILE, *const to2 = smem + 5 * K::TILE;  // dq (pass 1); dk, dv (pass 2)
    float *const den_all = reinterpret_cast<float *>(smem + OFF_DEN);
    float *const dden_all = reinterpret_cast<float *>(smem + OFF_DDEN);
    float *const part = reinterpret_cast<float *>(smem + OFF_PART);
    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = 16 * w + r, p0 = g * NP;   // layout A: column c, rows p0..; layout B: row c, columns p0..
    const size_t grp = blockIdx.x, tok0 = grp * (size_t)C;
    const uint32_t bytes = (uint32_t)C * D * sizeof(T);
    const GRes qr(q + tok0 * D, bytes), kr(k + tok0 * D, bytes), vr(v + tok0 * D, bytes), gr(dO + tok0 * D, bytes);
    const float *dummy = dS_in;
    const GRes sres(S_in ? (const void *)(S_in + grp * D * D) : dummy, S_in ? D * D * 4 : 0);
    const GRes zres(z_in ? (const void *)(z_in + grp * D) : dummy, z_in ? D * 4 : 0);
    const GRes shres(dS_out ? (const void *)(dS_out + grp * D * D) : dummy, dS_out ? D * D * 4 : 0);
    const GRes zhres(dz_out ? (const void *)(dz_out + grp * D) : dummy, dz_out ? D * 4 : 0);
    const int nbatch = (C + BT - 1) / BT;
    auto T_ = [](const char *tile) { return reinterpret_cast<const T *>(tile); };

    // layout A: SA[s] = S[p0 + s][c], zA[s] = z[p0 + s];  layout B: SB[s] = S[c][p0 + s], zB = z[c]
    float SA[NP], SB[NP], zA[NP], zB;
#pragma unroll
    for (int s = 0; s < NP; ++s) {
        SA[s] = gload<float>(sres, ((p0 + s) * D + c) * 4);
        SB[s] = gload<float>(sres, (c * D + p0 + s) * 4);
        zA[s] = gload<float>(zres, (p0 + s) * 4);
    }
    zB = gload<float>(zres, c * 4);
    Share<K::NV> sq, sk, sv, sg;
    auto load_batch = [&](int b) {  // b past the chunk (or negative offsets wrapped past it) read zeros
        const uint32_t off = b >= 0 ? (uint32_t)b * K::TILE : 0xF0000000u;
        sq.load(qr, off, tid);
        sk.load(kr, off, tid);
        sv.load(vr, off, tid);
        sg.load(gr, off, tid);
    };
    auto stage_batch = [&]() {
        __syncthreads();  // the previous batch's tiles are read and its outputs stored
        if constexpr (FM) {
            sq.template store_mapped<T>(tq, tid);
            sk.template store_mapped<T>(tk, tid);
        } else {
            sq.store(tq, tid);
            sk.store(tk, tid);
        }
        sv.store(tv, tid);
        sg.store(tg, tid);
        __syncthreads();
    };

    // ---- pass 1: tokens in order; den_t and dden_t kept for pass 2, dq stored
    load_batch(0);
    for (int b = 0; b < nbatch; ++b) {
        stage_batch();
        load_batch(b + 1 < nbatch ? b + 1 : nbatch - 1);  // pass 2 starts with the last batch
        const int n = C - b * BT < BT ? C - b * BT : BT;
        for (int t = 0; t < n; ++t) {
            const T *qt = T_(tq) + t * D, *kt = T_(tk) + t * D, *vt = T_(tv) + t * D, *gt = T_(tg) + t * D;
            const float vc = tof(vt[c]), kc = tof(kt[c]), gc = tof(gt[c]);
            float d[2] = {0.f, 0.f}, nn[2] = {0.f, 0.f};
#pragma unroll
            for (int s0 = 0; s0 < NP; s0 += 4) {
                const floatx4 kp = quad(kt + p0 + s0), qp = quad(qt + p0 + s0), vp = quad(vt + p0 + s0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = s0 + e;
                    zA[s] += kp[e];
                    SA[s] = __builtin_fmaf(kp[e], vc, SA[s]);
                    SB[s] = __builtin_fmaf(kc, vp[e], SB[s]);
                    d[e & 1] = __builtin_fmaf(qp[e], zA[s], d[e & 1]);
                    nn[e & 1] = __builtin_fmaf(qp[e], SA[s], nn[e & 1]);
                }
            }
            zB += kc;
            const float den = gsum(d[0] + d[1]), inv = 1.f / den;
            const float oc = gsum(nn[0] + nn[1]) * inv;
            // dO_t . o_t: over the wave's 16 columns, then over the waves
            float pd = gc * oc;
            pd += __shfl_xor(pd, 1);
            pd += __shfl_xor(pd, 2);
            pd += __shfl_xor(pd, 4);
            pd += __shfl_xor(pd, 8);
            if (lane == 0) part[(t & 1) * NW + w] = pd;
            __syncthreads();
            float rd = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) rd += part[(t & 1) * NW + ww];
            const float dden = -rd * inv;
            if (tid == 0) {
                den_all[b * BT + t] = den;
                dden_all[b * BT + t] = dden;
            }
            // dq[c] = sum over columns j of S[c][j] dO[j] / den + dden z[c]  (layout B, row c)
            float a[2] = {0.f, 0.f};
#pragma unroll
            for (int s0 = 0; s0 < NP; s0 += 4) {
                const floatx4 gp = quad(gt + p0 + s0);
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e & 1] = __builtin_fmaf(SB[s0 + e], gp[e], a[e & 1]);
            }
            float dqc = gsum(a[0] + a[1]) * inv + dden * zB;
            // fused feature map: the gradient of the raw input is dq phi'(x), phi' = min(1, phi)
            if constexpr (FM) dqc *= __builtin_fminf(tof(qt[c]), 1.f);
            if (g == 0) reinterpret_cast<T *>(to1)[t * D + c] = fromf<T>(dqc);
        }
        __syncthreads();
        flush_tile<T, D, K::NTH>(to1, dq + (tok0 + (size_t)b * BT) * D, n, tid);
    }

    // ---- pass 2: tokens in reverse, from the upstream carry gradient
#pragma unroll
    for (int s = 0; s < NP; ++s) {
        SA[s] = gload<float>(shres, ((p0 + s) * D + c) * 4);
        SB[s] = gload<float>(shres, (c * D + p0 + s) * 4);
    }
    zB = gload<float>(zhres, c * 4);
    for (int b = nbatch - 1; b >= 0; --b) {
        stage_batch();
        load_batch(b - 1);
        const int n = C - b * BT < BT ? C - b * BT : BT;
        for (int t = n - 1; t >= 0; --t) {
            const T *qt = T_(tq) + t * D, *kt = T_(tk) + t * D, *vt = T_(tv) + t * D, *gt = T_(tg) + t * D;
            const float inv = 1.f / den_all[b * BT + t], dden = dden_all[b * BT + t];
            const float dnc = tof(gt[c]) * inv, qc = tof(qt[c]);
            float a[2] = {0.f, 0.f}, x[2] = {0.f, 0.f};
            zB = __builtin_fmaf(dden, qc, zB);
#pragma unroll
            for (int s0 = 0; s0 < NP; s0 += 4) {
                const floatx4 kp = quad(kt + p0 + s0), qp = quad(qt + p0 + s0), vp = quad(vt + p0 + s0),
                              gp = quad(gt + p0 + s0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = s0 + e;
                    SA[s] = __builtin_fmaf(qp[e], dnc, SA[s]);          // Sh[p][c] += q[p] dn[c]
                    a[e & 1] = __builtin_fmaf(SA[s], kp[e], a[e & 1]);  // dv[c] = sum_p Sh[p][c] k[p]
                    SB[s] = __builtin_fmaf(qc, gp[e] * inv, SB[s]);     // Sh[c][j] += q[c] dn[j]
                    x[e & 1] = __builtin_fmaf(SB[s], vp[e], x[e & 1]);  // dk[c] = sum_j Sh[c][j] v[j] + zh[c]
                }
            }
            const float dvc = gsum(a[0] + a[1]);
            float dkc = gsum(x[0] + x[1]) + zB;
            if constexpr (FM) dkc *= __builtin_fminf(tof(kt[c]), 1.f);
            if (g == 0) {
                reinterpret_cast<T *>(to1)[t * D + c] = fromf<T>(dkc);
                reinterpret_cast<T *>(to2)[t * D + c] = fromf<T>(dvc);
            }
        }
        __syncthreads();
        flush_tile<T, D, K::NTH>(to1, dk + (tok0 + (size_t)b * BT) * D, n, tid);
        flush_tile<T, D, K::NTH>(to2, dv + (tok0 + (size_t)b * BT) * D, n, tid);
    }
#pragma unroll
    for (int s = 0; s < NP; ++s) dS_in[grp * D * D + (size_t)(p0 + s) * D + c] = SA[s];
    if (g == 0) dz_in[grp * D + c] = zB;
}

template <typename T, int D>
hipError_t launch_cumsum_fwd(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                             void *o, float *S_out, float *z_out, int G, int C, bool elu1, hipStream_t stream,
                             const hipEvent_t ev[2]) {
    hipExtLaunchKernelGGL(elu1 ? la_cumsum_fwd_kernel<T, D, true> : la_cumsum_fwd_kernel<T, D, false>,
                          dim3((unsigned)G), dim3(Cumsum<T, D>::NTH), 0, stream, ev[0], ev[1], 0, (const T *)q,
                          (const T *)k, (const T *)v, S_in, z_in, (T *)o, S_out, z_out, C);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_cumsum_bwd(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                             const void *dO, const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv,
                             float *dS_in, float *dz_in, int G, int C, bool elu1, hipStream_t stream,
                             const hipEvent_t ev[2]) {
    hipExtLaunchKernelGGL(elu1 ? la_cumsum_bwd_kernel<T, D, true> : la_cumsum_bwd_kernel<T, D, false>,
                          dim3((unsigned)G), dim3(Cumsum<T, D>::NTH), 0, stream, ev[0], ev[1], 0, (const T *)q,
                          (const T *)k, (const T *)v, S_in, z_in, (const T *)dO, dS_out, dz_out, (T *)dq, (T *)dk,
                          (T *)dv, dS_in, dz_in, C);
    return hipGetLastError();
}

#define LA_CUMSUM_INST(T, D)                                                                                        \
    template hipError_t launch_cumsum_fwd<T, D>(const void *, const void *, const void *, const float *,           \
                                                const float *, void *, float *, float *, int, int, bool,           \
                                                hipStream_t, const hipEvent_t *);                                   \
    template hipError_t launch_cumsum_bwd<T, D>(const void *, const void *, const void *, const float *,           \
                                                const float *, const void *, const float *, const float *, void *,  \
                                                void *, void *, float *, float *, int, int, bool, hipStream_t,      \
                                                const hipEvent_t *);
LA_CUMSUM_INST(float, 64)
LA_CUMSUM_INST(float, 128)
LA_CUMSUM_INST(__bf16, 64)
LA_CUMSUM_INST(__bf16, 128)

}  // namespace lachunk
