// Forward kernel: one chunk of causal linear attention with a carried state,
// blocked form ("Fractus-1B training optimization", section 2, Opt 2) with the
// exact per-token cumsum for the ragged tail.
//
// Grid: one workgroup per (group, 64-wide slice of value columns); 4 waves.
// Per 64-token block b, with the running state S_run (fp32: MFMA accumulators
// spread over the waves, mirrored in LDS) and z_run (LDS):
//   scores  P^T = K_b Q_b^T, masked to j <= t (inclusive)   [wave w: queries 16w..16w+15]
//   den_t   = sum_j P[t][j] + q_t . z_run                     [row sums by lane shuffles]
//   num^T   = V_b^T P^T + S_run^T Q_b^T                       [state read BEFORE the update]
//   o_t     = num_t / den_t
//   S_run  += K_b^T V_b,  z_run += K_b^T 1                    [update after reading]
// then the ragged tail token by token: S += k v^T, z += k, o = S^T q / (q . z).
// P and S_run enter the MFMAs as bf16 hi + lo pairs (see la_common.h).
#include "la_common.h"
#include "la_launch.h"

namespace lachunk {

template <typename T, int D>
struct FwdLds {
    static constexpr int PAD = Elem<T>::PAD;
    static constexpr int LDN = D + PAD;    // token-major rows (k = feature)
    static constexpr int LDT = BK + PAD;   // feature-major rows (k = token)
    static constexpr int LDSF = 64 + 4;    // fp32 state slice S[p][c], 64 value columns
    static constexpr int ZS = 0;                                        // [D] z_run
    static constexpr int SF = ((D * 4 + 15) / 16) * 16;                 // [D][LDSF] fp32
    static constexpr int BASE = SF + D * LDSF * 4;
    // block phase
    static constexpr int KN = BASE;                                     // [BK][LDN] K
    static constexpr int KT = KN + BK * LDN * (int)sizeof(T);           // [D][LDT]  K^T
    static constexpr int VT = KT + D * LDT * (int)sizeof(T);            // [64][LDT] V^T (slice)
    static constexpr int BLOCK_END = VT + 64 * LDT * (int)sizeof(T);
    // ragged-tail phase
    static constexpr int TQ = BASE;                                     // [BK][LDN] q
    static constexpr int TK = TQ + BK * LDN * (int)sizeof(T);           // [BK][LDN] k
    static constexpr int TV = TK + BK * LDN * (int)sizeof(T);           // [BK][LDT] v (slice)
    static constexpr int TAIL_END = TV + BK * LDT * (int)sizeof(T);
    static constexpr int BYTES = BLOCK_END > TAIL_END ? BLOCK_END : TAIL_END;
    static_assert(BYTES <= 160 * 1024, "forward LDS budget exceeded");
};

template <typename T, int D>
__global__ __launch_bounds__(NTHR, 1) void la_fwd_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in,
    T *__restrict__ o, float *__restrict__ S_out, float *__restrict__ z_out, int C) {
    using L = FwdLds<T, D>;
    constexpr int NVS = D / 64;          // value slices per group
    constexpr int NPT = D / 16 / NWAVE;  // key-feature tiles of the state per wave
    constexpr int NKC = D / 32;          // k-chunks over the feature dimension
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    float *zs = reinterpret_cast<float *>(smem + L::ZS);
    float *Sf = reinterpret_cast<float *>(smem + L::SF);
    T *Kn = reinterpret_cast<T *>(smem + L::KN);
    T *Kt = reinterpret_cast<T *>(smem + L::KT);
    T *Vt = reinterpret_cast<T *>(smem + L::VT);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
    const int grp = blockIdx.x / NVS, vs = blockIdx.x % NVS;
    const size_t tok0 = (size_t)grp * C;
    const T *qg = q + tok0 * D;
    const T *kg = k + tok0 * D;
    const T *vg = v + tok0 * D;
    T *og = o + tok0 * D;
    const int nb = C / BK, tail = C % BK;

    // ---- issue every load the first block needs before waiting on any of them
    F32Tile<D, 64> sin;
    sin.load(S_in ? S_in + (size_t)grp * D * D + vs * 64 : nullptr, D, tid);
    const float zin = (tid < D && z_in) ? z_in[(size_t)grp * D + tid] : 0.f;
    Stager<T, D> kst;
    Stager<T, 64> vst;
    Frag<T> qf[NKC];
    if (nb > 0) {
        kst.load(kg, D, BK, tid);
        vst.load(vg + vs * 64, D, BK, tid);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) qf[kc] = ldfrag<T>(qg + (size_t)(16 * w) * D + 32 * kc, D, lane);
    }
    sin.store(Sf, L::LDSF, tid);
    if (tid < D) zs[tid] = zin;
    __syncthreads();

    // state accumulators acc(p, c) of this value slice; wave w owns p-tiles w + 4*pi
    floatx4 Sacc[NPT][4];
#pragma unroll
    for (int pi = 0; pi < NPT; ++pi)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) Sacc[pi][ct][i] = Sf[(16 * (w + 4 * pi) + 4 * g + i) * L::LDSF + 16 * ct + r];

    const Frag<T> ones = ones_frag<T>();
    for (int b = 0; b < nb; ++b) {
        const int t0 = b * BK;
        if (b > 0) __syncthreads();  // previous block's update of Sf / zs is complete; staging arrays free
        kst.store(Kn, L::LDN, Kt, L::LDT, tid);
        vst.store(nullptr, 0, Vt, L::LDT, tid);
        Frag<T> qc[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) qc[kc] = qf[kc];
        if (b + 1 < nb) {  // prefetch the next block while this one computes
            kst.load(kg + (size_t)(t0 + BK) * D, D, BK, tid);
            vst.load(vg + (size_t)(t0 + BK) * D + vs * 64, D, BK, tid);
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) qf[kc] = ldfrag<T>(qg + (size_t)(t0 + BK + 16 * w) * D + 32 * kc, D, lane);
        }
        __syncthreads();

        // scores P^T[j][t] for key tiles jt <= w (later tiles are fully masked)
        floatx4 sc[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            sc[jt] = zero4();
            if (jt <= w) {
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) mma(sc[jt], ldfrag<T>(Kn + 16 * jt * L::LDN + 32 * kc, L::LDN, lane), qc[kc]);
            }
            if (jt == w) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * g + i > r) sc[jt][i] = 0.f;  // key after query
            }
        }
        // den_t = sum_j P[t][j] + q_t . z_run
        float dsum = 0.f;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i) dsum += sc[jt][i];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
            for (int s = 0; s < 8; ++s) dsum += tof(qc[kc][s]) * zs[32 * kc + kslot(lane, s)];
        dsum = wsum_g(dsum);
        const float inv = 1.f / dsum;

        // num^T[c][t] = V^T P^T (intra) + S_run^T Q^T (inter, state before this block)
        const SFrag<T> pf0 = split8<T>(acc8(sc[0], sc[1]));
        const SFrag<T> pf1 = split8<T>(acc8(sc[2], sc[3]));
        T *orow = og + (size_t)(t0 + 16 * w + r) * D + vs * 64 + 4 * g;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            floatx4 nm = zero4();
            mma_xs<T>(nm, ldfrag<T>(Vt + 16 * ct * L::LDT, L::LDT, lane), pf0);
            if (w >= 2) mma_xs<T>(nm, ldfrag<T>(Vt + 16 * ct * L::LDT + 32, L::LDT, lane), pf1);
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
                mma_sx<T>(nm, split8<T>(ld8_cols(Sf + 32 * kc * L::LDSF + 16 * ct, L::LDSF, lane)), qc[kc]);
            *reinterpret_cast<Vec4<T> *>(orow + 16 * ct) = to_vec4<T>(nm * inv);
        }
        __syncthreads();  // every wave is done reading Sf, Vt and zs for this block

        // update after reading: S_run += K^T V, z_run += K^T 1
#pragma unroll
        for (int pi = 0; pi < NPT; ++pi) {
            const int p0 = 16 * (w + 4 * pi);
            const Frag<T> kf0 = ldfrag<T>(Kt + p0 * L::LDT, L::LDT, lane);
            const Frag<T> kf1 = ldfrag<T>(Kt + p0 * L::LDT + 32, L::LDT, lane);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                mma(Sacc[pi][ct], kf0, ldfrag<T>(Vt + 16 * ct * L::LDT, L::LDT, lane));
                mma(Sacc[pi][ct], kf1, ldfrag<T>(Vt + 16 * ct * L::LDT + 32, L::LDT, lane));
#pragma unroll
                for (int i = 0; i < 4; ++i) Sf[(p0 + 4 * g + i) * L::LDSF + 16 * ct + r] = Sacc[pi][ct][i];
            }
            floatx4 zacc = zero4();
            mma(zacc, kf0, ones);
            mma(zacc, kf1, ones);
            if (r == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) zs[p0 + 4 * g + i] += zacc[i];
            }
        }
    }

    if (tail == 0) {
        float *Sg = S_out + (size_t)grp * D * D + vs * 64;
#pragma unroll
        for (int pi = 0; pi < NPT; ++pi)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Sg[(size_t)(16 * (w + 4 * pi) + 4 * g + i) * D + 16 * ct + r] = Sacc[pi][ct][i];
        __syncthreads();
        if (vs == 0 && tid < D) z_out[(size_t)grp * D + tid] = zs[tid];
        return;
    }

    // ---- ragged tail: exact per-token cumsum from (S_run, z_run)
    T *Tq = reinterpret_cast<T *>(smem + L::TQ);
    T *Tk = reinterpret_cast<T *>(smem + L::TK);
    T *Tv = reinterpret_cast<T *>(smem + L::TV);
    const int tt0 = nb * BK;
    {
        Stager<T, D> qs, ks;
        Stager<T, 64> vs_;
        qs.load(qg + (size_t)tt0 * D, D, tail, tid);
        ks.load(kg + (size_t)tt0 * D, D, tail, tid);
        vs_.load(vg + (size_t)tt0 * D + vs * 64, D, tail, tid);
        __syncthreads();  // the block phase is finished with every staging array
        qs.store(Tq, L::LDN, nullptr, 0, tid);
        ks.store(Tk, L::LDN, nullptr, 0, tid);
        vs_.store(Tv, L::LDT, nullptr, 0, tid);
        __syncthreads();
    }
    // lane owns value column c = 16w + r of the slice and key features p in [g*NP, (g+1)*NP)
    constexpr int NP = D / 4;
    const int c = 16 * w + r;
    float Sr[NP], zr[NP];
#pragma unroll
    for (int s = 0; s < NP; ++s) {
        Sr[s] = Sf[(g * NP + s) * L::LDSF + c];
        zr[s] = zs[g * NP + s];
    }
    for (int t = 0; t < tail; ++t) {
        const float vc = tof(Tv[t * L::LDT + c]);
        const T *kt = Tk + t * L::LDN + g * NP;
        const T *qt = Tq + t * L::LDN + g * NP;
        float n = 0.f, d = 0.f;
#pragma unroll
        for (int s4 = 0; s4 < NP; s4 += 4) {
            const Vec4<T> k4 = *reinterpret_cast<const Vec4<T> *>(kt + s4);
            const Vec4<T> q4 = *reinterpret_cast<const Vec4<T> *>(qt + s4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float kp = tof(k4[e]), qp = tof(q4[e]);
                Sr[s4 + e] += kp * vc;  // update first: token t reads a state that includes it
                zr[s4 + e] += kp;
                n += qp * Sr[s4 + e];
                d += qp * zr[s4 + e];
            }
        }
        n = wsum_g(n);
        d = wsum_g(d);
        if (g == 0) og[(size_t)(tt0 + t) * D + vs * 64 + c] = fromf<T>(n / d);
    }
    float *Sg = S_out + (size_t)grp * D * D + vs * 64;
#pragma unroll
    for (int s = 0; s < NP; ++s) Sg[(size_t)(g * NP + s) * D + c] = Sr[s];
    if (vs == 0 && w == 0 && r == 0) {
#pragma unroll
        for (int s = 0; s < NP; ++s) z_out[(size_t)grp * D + g * NP + s] = zr[s];
    }
}

template <typename T, int D>
hipError_t launch_fwd(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                      void *o, float *S_out, float *z_out, int G, int C, hipStream_t stream) {
    dim3 grid((unsigned)G * (D / 64)), block(NTHR);
    hipLaunchKernelGGL((la_fwd_kernel<T, D>), grid, block, 0, stream,
                       (const T *)q, (const T *)k, (const T *)v, S_in, z_in, (T *)o, S_out, z_out, C);
    return hipGetLastError();
}

template hipError_t launch_fwd<float, 64>(const void *, const void *, const void *, const float *, const float *,
                                          void *, float *, float *, int, int, hipStream_t);
template hipError_t launch_fwd<float, 128>(const void *, const void *, const void *, const float *, const float *,
                                           void *, float *, float *, int, int, hipStream_t);
template hipError_t launch_fwd<bf16, 64>(const void *, const void *, const void *, const float *, const float *,
                                         void *, float *, float *, int, int, hipStream_t);
template hipError_t launch_fwd<bf16, 128>(const void *, const void *, const void *, const float *, const float *,
                                          void *, float *, float *, int, int, hipStream_t);

}  // namespace lachunk
