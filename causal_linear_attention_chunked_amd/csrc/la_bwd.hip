// Backward kernel: reverse scan for one chunk ("Fractus-1B training
// optimization", section 1: the gradient of a prefix sum is a suffix sum, not
// another masked matmul).  It recomputes the forward from its inputs.
//
// Loss L = sum_t <dO_t, o_t> + <dS_out, S_out> + dz_out . z_out.  Per token,
//   den_t = q_t . z_t,  dn_t = dO_t / den_t,  dden_t = -(dO_t . o_t) / den_t,
//   dq_t = S_t dn_t + dden_t z_t,
//   Sh_t = dS_out + sum_{i>=t} q_i dn_i^T,  zh_t = dz_out + sum_{i>=t} dden_i q_i,
//   dk_t = Sh_t v_t + zh_t,  dv_t = Sh_t^T k_t,  dS_in = Sh_1,  dz_in = zh_1.
// In 64-token blocks (A = Q K^T masked inclusively, S_b / z_b the state before
// block b, Sh / zh the reverse state holding every later token):
//   pass 1, blocks in order:  den, o (recomputed), dN, dden;
//                             dP = (dN V^T + dden 1^T) masked;  dQ = dP K + dN S_b^T + dden z_b^T;
//                             S_b += K^T V,  z_b += K^T 1
//   pass 2, blocks reversed:  dV = A^T dN + K Sh;   dK = dP^T Q + V Sh^T + 1 zh^T;
//                             Sh += Q^T dN,  zh += Q^T dden
// The ragged tail runs token by token: last in pass 1, first in pass 2.
// Grid: one workgroup per group, 4 waves.  Every fp32 intermediate (P, dP, dN,
// dden, S, Sh) enters the MFMAs as a bf16 hi + lo pair (see la_common.h); the
// state lives once in LDS as fp32 and in the waves' accumulators.
#include "la_common.h"
#include "la_launch.h"
#include "../../include/la_chunk.h"

namespace lachunk {

template <typename T, int D>
struct BwdLds {
    static constexpr int PAD = Elem<T>::PAD;
    static constexpr int LDN = D + PAD;   // token-major rows (k = feature)
    static constexpr int LDT = BK + PAD;  // feature-major rows (k = token)
    static constexpr int LDSF = D + 4;    // fp32 state S[p][c]
    static constexpr int CMAX = LA_BWD_MAX_C;
    static constexpr int ZS = 0;                                  // [D] z_b (pass 1) / zh (pass 2)
    static constexpr int DEN = ZS + D * 4;                        // [CMAX] den_t
    static constexpr int DDEN = DEN + CMAX * 4;                   // [CMAX] dden_t
    static constexpr int PART = DDEN + CMAX * 4;                  // [2][NWAVE] tail row-dot partials
    static constexpr int SF = ((PART + 2 * NWAVE * 4 + 15) / 16) * 16;   // [D][LDSF] state, fp32
    static constexpr int BASE = SF + D * LDSF * 4;
    // block phase (pass 1 names / pass 2 names)
    static constexpr int N0 = BASE;                                   // K  / Q   [BK][LDN]
    static constexpr int N1 = N0 + BK * LDN * (int)sizeof(T);         // V  / dO  [BK][LDN]
    static constexpr int T0 = N1 + BK * LDN * (int)sizeof(T);         // K^T / Q^T  [D][LDT]
    static constexpr int T1 = T0 + D * LDT * (int)sizeof(T);          // V^T / dO^T [D][LDT]
    static constexpr int BLOCK_END = T1 + D * LDT * (int)sizeof(T);
    // ragged-tail phase: q, k, v, dO rows
    static constexpr int TQ = BASE;
    static constexpr int TK = TQ + BK * LDN * (int)sizeof(T);
    static constexpr int TV = TK + BK * LDN * (int)sizeof(T);
    static constexpr int TG = TV + BK * LDN * (int)sizeof(T);
    static constexpr int TAIL_END = TG + BK * LDN * (int)sizeof(T);
    static constexpr int BYTES = BLOCK_END > TAIL_END ? BLOCK_END : TAIL_END;
    static_assert(BYTES <= 160 * 1024, "backward LDS budget exceeded");
};

template <typename T, int D>
__global__ __launch_bounds__(NTHR, 1) void la_bwd_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in, const T *__restrict__ dO,
    const float *__restrict__ dS_out, const float *__restrict__ dz_out,
    T *__restrict__ dq, T *__restrict__ dk, T *__restrict__ dv,
    float *__restrict__ dS_in, float *__restrict__ dz_in, int C) {
    using L = BwdLds<T, D>;
    constexpr int NPT = D / 16 / NWAVE;  // state row tiles per wave
    constexpr int NCT = D / 16;          // feature tiles
    constexpr int NKC = D / 32;          // k-chunks over the feature dimension
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    float *zs = reinterpret_cast<float *>(smem + L::ZS);
    float *den_all = reinterpret_cast<float *>(smem + L::DEN);
    float *dden_all = reinterpret_cast<float *>(smem + L::DDEN);
    float *part = reinterpret_cast<float *>(smem + L::PART);
    float *Sf = reinterpret_cast<float *>(smem + L::SF);
    T *N0 = reinterpret_cast<T *>(smem + L::N0);
    T *N1 = reinterpret_cast<T *>(smem + L::N1);
    T *T0 = reinterpret_cast<T *>(smem + L::T0);
    T *T1 = reinterpret_cast<T *>(smem + L::T1);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
    const int grp = blockIdx.x;
    const size_t tok0 = (size_t)grp * C;
    const T *qg = q + tok0 * D, *kg = k + tok0 * D, *vg = v + tok0 * D, *gg = dO + tok0 * D;
    T *dqg = dq + tok0 * D, *dkg = dk + tok0 * D, *dvg = dv + tok0 * D;
    const int nb = C / BK, tail = C % BK, tt0 = nb * BK;
    const Frag<T> ones = ones_frag<T>();

    // state accumulators acc(p, c): wave w owns row tiles w + 4*pi, every column tile
    floatx4 Sacc[NPT][NCT];
    auto sf_to_acc = [&]() {
#pragma unroll
        for (int pi = 0; pi < NPT; ++pi)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Sacc[pi][ct][i] = Sf[(16 * (w + 4 * pi) + 4 * g + i) * L::LDSF + 16 * ct + r];
    };

    // ---- pass 1 prologue: state, normaliser and the first block, all loads in flight together
    F32Tile<D, D> stile;
    stile.load(S_in ? S_in + (size_t)grp * D * D : nullptr, D, tid);
    const float zin = (tid < D && z_in) ? z_in[(size_t)grp * D + tid] : 0.f;
    Stager<T, D> st0, st1;
    Frag<T> qf[NKC], kf[NKC], vf[NKC];
    Vec4<T> gv[NCT];
    auto load_pass1 = [&](int t0) {
        st0.load(kg + (size_t)t0 * D, D, BK, tid);
        st1.load(vg + (size_t)t0 * D, D, BK, tid);
        const size_t row = (size_t)(t0 + 16 * w);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) qf[kc] = ldfrag<T>(qg + row * D + 32 * kc, D, lane);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            gv[ct] = *reinterpret_cast<const Vec4<T> *>(gg + (row + r) * D + 16 * ct + 4 * g);
    };
    auto load_pass2 = [&](int t0) {
        st0.load(qg + (size_t)t0 * D, D, BK, tid);
        st1.load(gg + (size_t)t0 * D, D, BK, tid);
        const size_t row = (size_t)(t0 + 16 * w);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            kf[kc] = ldfrag<T>(kg + row * D + 32 * kc, D, lane);
            vf[kc] = ldfrag<T>(vg + row * D + 32 * kc, D, lane);
        }
    };
    if (nb > 0) load_pass1(0);
    stile.store(Sf, L::LDSF, tid);
    if (tid < D) zs[tid] = zin;
    __syncthreads();
    sf_to_acc();

    // =========================== pass 1: forward sweep ===========================
    for (int b = 0; b < nb; ++b) {
        const int t0 = b * BK;
        T *Kn = N0, *Vn = N1, *Kt = T0, *Vt = T1;
        if (b > 0) __syncthreads();  // the previous block's state update is visible; staging arrays free
        st0.store(Kn, L::LDN, Kt, L::LDT, tid);
        st1.store(Vn, L::LDN, Vt, L::LDT, tid);
        Frag<T> qc[NKC];
        Vec4<T> gc[NCT];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) qc[kc] = qf[kc];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) gc[ct] = gv[ct];
        if (b + 1 < nb) load_pass1(t0 + BK);
        else if (tail == 0) load_pass2(t0);  // pass 2 starts on this same block
        __syncthreads();

        const int trow = t0 + 16 * w + r;
        // scores P^T[j][t] (lane: query t = 16w + r, keys 4g+i of tile jt)
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
                    if (4 * g + i > r) sc[jt][i] = 0.f;
            }
        }
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

        // o (recomputed), then dN = dO / den (kept as acc(c, t)) and dden = -(dO . o) / den
        floatx4 dN[NCT];
        float rowdot = 0.f;
        {
            const SFrag<T> pf0 = split8<T>(acc8(sc[0], sc[1]));
            const SFrag<T> pf1 = split8<T>(acc8(sc[2], sc[3]));
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                floatx4 nm = zero4();
                mma_xs<T>(nm, ldfrag<T>(Vt + 16 * ct * L::LDT, L::LDT, lane), pf0);
                if (w >= 2) mma_xs<T>(nm, ldfrag<T>(Vt + 16 * ct * L::LDT + 32, L::LDT, lane), pf1);
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc)
                    mma_sx<T>(nm, split8<T>(ld8_cols(Sf + 32 * kc * L::LDSF + 16 * ct, L::LDSF, lane)), qc[kc]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float gi = tof(gc[ct][i]);
                    rowdot += gi * nm[i];
                    dN[ct][i] = gi * inv;
                }
            }
        }
        rowdot = wsum_g(rowdot);
        const float dden = -rowdot * inv * inv;
        if (g == 0) {
            den_all[trow] = dsum;
            dden_all[trow] = dden;
        }
        SFrag<T> dNs[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) dNs[kc] = split8<T>(acc8(dN[2 * kc], dN[2 * kc + 1]));

        // dP^T[j][t] = sum_c V[j][c] dN[t][c] + dden_t, masked j <= t
        floatx4 dp[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            dp[jt] = zero4();
            if (jt <= w) {
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc)
                    mma_xs<T>(dp[jt], ldfrag<T>(Vn + 16 * jt * L::LDN + 32 * kc, L::LDN, lane), dNs[kc]);
#pragma unroll
                for (int i = 0; i < 4; ++i) dp[jt][i] += dden;
            }
            if (jt == w) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * g + i > r) dp[jt][i] = 0.f;
            }
        }
        // dQ^T[p][t] = K^T dP^T + S_b dN^T + z_b dden
        {
            const SFrag<T> df0 = split8<T>(acc8(dp[0], dp[1]));
            const SFrag<T> df1 = split8<T>(acc8(dp[2], dp[3]));
            T *drow = dqg + (size_t)trow * D + 4 * g;
#pragma unroll
            for (int pt = 0; pt < NCT; ++pt) {
                floatx4 a = zero4();
                mma_xs<T>(a, ldfrag<T>(Kt + 16 * pt * L::LDT, L::LDT, lane), df0);
                if (w >= 2) mma_xs<T>(a, ldfrag<T>(Kt + 16 * pt * L::LDT + 32, L::LDT, lane), df1);
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc)
                    mma_ss<T>(a, split8<T>(ld8_rows(Sf + 16 * pt * L::LDSF + 32 * kc, L::LDSF, lane)), dNs[kc]);
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] += dden * zs[16 * pt + 4 * g + i];
                *reinterpret_cast<Vec4<T> *>(drow + 16 * pt) = to_vec4<T>(a);
            }
        }
        if (b + 1 == nb && tail == 0) break;  // the state after the last block is not needed
        __syncthreads();
        // S_b += K^T V, z_b += K^T 1
#pragma unroll
        for (int pi = 0; pi < NPT; ++pi) {
            const int p0 = 16 * (w + 4 * pi);
            const Frag<T> kf0 = ldfrag<T>(Kt + p0 * L::LDT, L::LDT, lane);
            const Frag<T> kf1 = ldfrag<T>(Kt + p0 * L::LDT + 32, L::LDT, lane);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
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

    // =========================== ragged tail (both passes) ===========================
    constexpr int NP = D / 4;     // features per lane-group
    constexpr int NH = D / 64;    // columns (layout A) / rows (layout B) per lane
    bool sh_zero = false;         // the reverse state is known to be exactly zero
    if (tail > 0) {
        T *Tq = reinterpret_cast<T *>(smem + L::TQ);
        T *Tk = reinterpret_cast<T *>(smem + L::TK);
        T *Tv = reinterpret_cast<T *>(smem + L::TV);
        T *Tg = reinterpret_cast<T *>(smem + L::TG);
        {
            Stager<T, D> a, b2, c2, d2;
            a.load(qg + (size_t)tt0 * D, D, tail, tid);
            b2.load(kg + (size_t)tt0 * D, D, tail, tid);
            c2.load(vg + (size_t)tt0 * D, D, tail, tid);
            d2.load(gg + (size_t)tt0 * D, D, tail, tid);
            __syncthreads();
            a.store(Tq, L::LDN, nullptr, 0, tid);
            b2.store(Tk, L::LDN, nullptr, 0, tid);
            c2.store(Tv, L::LDN, nullptr, 0, tid);
            d2.store(Tg, L::LDN, nullptr, 0, tid);
            __syncthreads();
        }
        // layout A: lane owns columns cA[h] = 64h + 16w + r, key features g*NP.. (as rows p)
        // layout B: lane owns rows pB[h] = 64h + 16w + r, value features g*NP.. (as columns c)
        float SA[NH][NP], SB[NH][NP], zA[NP], zB[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int s = 0; s < NP; ++s) {
                SA[h][s] = Sf[(g * NP + s) * L::LDSF + 64 * h + 16 * w + r];
                SB[h][s] = Sf[(64 * h + 16 * w + r) * L::LDSF + g * NP + s];
            }
#pragma unroll
        for (int s = 0; s < NP; ++s) zA[s] = zs[g * NP + s];
#pragma unroll
        for (int h = 0; h < NH; ++h) zB[h] = zs[64 * h + 16 * w + r];

        // ---- pass 1 tail: forward order
        for (int t = 0; t < tail; ++t) {
            const T *qt = Tq + t * L::LDN, *kt = Tk + t * L::LDN, *vt = Tv + t * L::LDN, *gt = Tg + t * L::LDN;
            float n[NH], d = 0.f, vA[NH];
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                n[h] = 0.f;
                vA[h] = tof(vt[64 * h + 16 * w + r]);
            }
#pragma unroll
            for (int s = 0; s < NP; ++s) {
                const float kp = tof(kt[g * NP + s]), qp = tof(qt[g * NP + s]);
                zA[s] += kp;
                d += qp * zA[s];
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    SA[h][s] += kp * vA[h];
                    n[h] += qp * SA[h][s];
                }
            }
            d = wsum_g(d);
            const float inv = 1.f / d;
            float pd = 0.f;
#pragma unroll
            for (int h = 0; h < NH; ++h) pd += tof(gt[64 * h + 16 * w + r]) * (wsum_g(n[h]) * inv);
            pd += __shfl_xor(pd, 1);
            pd += __shfl_xor(pd, 2);
            pd += __shfl_xor(pd, 4);
            pd += __shfl_xor(pd, 8);
            if (lane == 0) part[(t & 1) * NWAVE + w] = pd;
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const float kp = tof(kt[64 * h + 16 * w + r]);
                zB[h] += kp;
#pragma unroll
                for (int s = 0; s < NP; ++s) SB[h][s] += kp * tof(vt[g * NP + s]);
            }
            __syncthreads();
            float rd = 0.f;
#pragma unroll
            for (int ww = 0; ww < NWAVE; ++ww) rd += part[(t & 1) * NWAVE + ww];
            const float ddn = -rd * inv;
            if (tid == 0) {
                den_all[tt0 + t] = d;
                dden_all[tt0 + t] = ddn;
            }
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                float a = 0.f;
#pragma unroll
                for (int s = 0; s < NP; ++s) a += SB[h][s] * tof(gt[g * NP + s]);
                a = wsum_g(a) * inv + ddn * zB[h];
                if (g == 0) dqg[(size_t)(tt0 + t) * D + 64 * h + 16 * w + r] = fromf<T>(a);
            }
        }

        // ---- pass 2 tail: reverse order, from the upstream carry gradient
        const float *dSo = dS_out ? dS_out + (size_t)grp * D * D : nullptr;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
#pragma unroll
            for (int s = 0; s < NP; ++s) {
                SA[h][s] = dSo ? dSo[(size_t)(g * NP + s) * D + 64 * h + 16 * w + r] : 0.f;
                SB[h][s] = dSo ? dSo[(size_t)(64 * h + 16 * w + r) * D + g * NP + s] : 0.f;
            }
            zB[h] = dz_out ? dz_out[(size_t)grp * D + 64 * h + 16 * w + r] : 0.f;
        }
        __syncthreads();  // den_all / dden_all of the tail are visible
        for (int t = tail - 1; t >= 0; --t) {
            const T *qt = Tq + t * L::LDN, *kt = Tk + t * L::LDN, *vt = Tv + t * L::LDN, *gt = Tg + t * L::LDN;
            const float inv = 1.f / den_all[tt0 + t], ddn = dden_all[tt0 + t];
            float dnA[NH], a[NH];
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                dnA[h] = tof(gt[64 * h + 16 * w + r]) * inv;
                a[h] = 0.f;
            }
#pragma unroll
            for (int s = 0; s < NP; ++s) {
                const float qp = tof(qt[g * NP + s]), kp = tof(kt[g * NP + s]);
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    SA[h][s] += qp * dnA[h];
                    a[h] += SA[h][s] * kp;
                }
            }
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const float x = wsum_g(a[h]);
                if (g == 0) dvg[(size_t)(tt0 + t) * D + 64 * h + 16 * w + r] = fromf<T>(x);
            }
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const float qp = tof(qt[64 * h + 16 * w + r]);
                zB[h] += ddn * qp;
                float x = 0.f;
#pragma unroll
                for (int s = 0; s < NP; ++s) {
                    SB[h][s] += qp * (tof(gt[g * NP + s]) * inv);
                    x += SB[h][s] * tof(vt[g * NP + s]);
                }
                x = wsum_g(x) + zB[h];
                if (g == 0) dkg[(size_t)(tt0 + t) * D + 64 * h + 16 * w + r] = fromf<T>(x);
            }
        }
        if (nb == 0) {
            float *dSg = dS_in + (size_t)grp * D * D;
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int s = 0; s < NP; ++s) dSg[(size_t)(g * NP + s) * D + 64 * h + 16 * w + r] = SA[h][s];
            if (g == 0) {
#pragma unroll
                for (int h = 0; h < NH; ++h) dz_in[(size_t)grp * D + 64 * h + 16 * w + r] = zB[h];
            }
            return;
        }
        load_pass2((nb - 1) * BK);
        __syncthreads();  // every wave is done with Sf and zs of pass 1
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int s = 0; s < NP; ++s) Sf[(g * NP + s) * L::LDSF + 64 * h + 16 * w + r] = SA[h][s];
        if (g == 0) {
#pragma unroll
            for (int h = 0; h < NH; ++h) zs[64 * h + 16 * w + r] = zB[h];
        }
    } else {
        // no tail: the reverse state starts at the upstream carry gradient
        sh_zero = dS_out == nullptr;
        stile.load(dS_out ? dS_out + (size_t)grp * D * D : nullptr, D, tid);
        const float dzo = (tid < D && dz_out) ? dz_out[(size_t)grp * D + tid] : 0.f;
        __syncthreads();  // pass 1 is done reading Sf and zs
        stile.store(Sf, L::LDSF, tid);
        if (tid < D) zs[tid] = dzo;
    }
    __syncthreads();
    sf_to_acc();

    // =========================== pass 2: reverse sweep over blocks ===========================
    for (int b = nb - 1; b >= 0; --b) {
        const int t0 = b * BK;
        T *Qn = N0, *Gn = N1, *Qt = T0, *Gt = T1;
        if (b < nb - 1) __syncthreads();
        st0.store(Qn, L::LDN, Qt, L::LDT, tid);
        st1.store(Gn, L::LDN, Gt, L::LDT, tid);
        Frag<T> kc_[NKC], vc_[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            kc_[kc] = kf[kc];
            vc_[kc] = vf[kc];
        }
        if (b > 0) load_pass2(t0 - BK);
        // per-slot 1/den_t and dden_t of the two 32-token chunks (slot s of chunk h: t = 32h + kslot)
        floatx8 isc[2], dsl[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int t = t0 + 32 * h + kslot(lane, s);
                isc[h][s] = 1.f / den_all[t];
                dsl[h][s] = dden_all[t];
            }
        __syncthreads();

        // P[t][j] and dP[t][j] as acc(t, j): lane holds key j = 16w + r, queries 16tt + 4g + i
        floatx4 ap[4], ad[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            ap[tt] = zero4();
            ad[tt] = zero4();
            if (tt >= w) {
                const float sc_row = 1.f / den_all[t0 + 16 * tt + r];
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) {
                    mma(ap[tt], ldfrag<T>(Qn + 16 * tt * L::LDN + 32 * kc, L::LDN, lane), kc_[kc]);
                    mma_sx<T>(ad[tt], split8<T>(ld8_scaled<T>(Gn + 16 * tt * L::LDN + 32 * kc, L::LDN, lane, sc_row)),
                              vc_[kc]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) ad[tt][i] += dden_all[t0 + 16 * tt + 4 * g + i];
            }
            if (tt == w) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (r > 4 * g + i) {  // key after query
                        ap[tt][i] = 0.f;
                        ad[tt][i] = 0.f;
                    }
            }
        }
        // dV^T[c][j] = dN^T P (intra) + Sh^T K^T (inter);   dK^T[p][j] = Q^T dP (intra) + Sh V^T + zh
        {
            const SFrag<T> pa0 = split8<T>(acc8(ap[0], ap[1])), pa1 = split8<T>(acc8(ap[2], ap[3]));
            const SFrag<T> pd0 = split8<T>(acc8(ad[0], ad[1])), pd1 = split8<T>(acc8(ad[2], ad[3]));
            const int jrow = t0 + 16 * w + r;
            T *vrow = dvg + (size_t)jrow * D + 4 * g;
            T *krow = dkg + (size_t)jrow * D + 4 * g;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                floatx4 a = zero4();
                if (w < 2) mma_ss<T>(a, split8<T>(ld8_scaled<T>(Gt + 16 * ct * L::LDT, L::LDT, lane, isc[0])), pa0);
                mma_ss<T>(a, split8<T>(ld8_scaled<T>(Gt + 16 * ct * L::LDT + 32, L::LDT, lane, isc[1])), pa1);
                if (!sh_zero) {
#pragma unroll
                    for (int kc = 0; kc < NKC; ++kc)
                        mma_sx<T>(a, split8<T>(ld8_cols(Sf + 32 * kc * L::LDSF + 16 * ct, L::LDSF, lane)), kc_[kc]);
                }
                *reinterpret_cast<Vec4<T> *>(vrow + 16 * ct) = to_vec4<T>(a);
            }
#pragma unroll
            for (int pt = 0; pt < NCT; ++pt) {
                floatx4 a = zero4();
                if (w < 2) mma_xs<T>(a, ldfrag<T>(Qt + 16 * pt * L::LDT, L::LDT, lane), pd0);
                mma_xs<T>(a, ldfrag<T>(Qt + 16 * pt * L::LDT + 32, L::LDT, lane), pd1);
                if (!sh_zero) {
#pragma unroll
                    for (int kc = 0; kc < NKC; ++kc)
                        mma_sx<T>(a, split8<T>(ld8_rows(Sf + 16 * pt * L::LDSF + 32 * kc, L::LDSF, lane)), vc_[kc]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) a[i] += zs[16 * pt + 4 * g + i];
                }
                *reinterpret_cast<Vec4<T> *>(krow + 16 * pt) = to_vec4<T>(a);
            }
        }
        __syncthreads();
        // Sh += Q^T dN, zh += Q^T dden
        const SFrag<T> dd0 = split8<T>(dsl[0]), dd1 = split8<T>(dsl[1]);
#pragma unroll
        for (int pi = 0; pi < NPT; ++pi) {
            const int p0 = 16 * (w + 4 * pi);
            const Frag<T> qa = ldfrag<T>(Qt + p0 * L::LDT, L::LDT, lane);
            const Frag<T> qb = ldfrag<T>(Qt + p0 * L::LDT + 32, L::LDT, lane);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                mma_xs<T>(Sacc[pi][ct], qa, split8<T>(ld8_scaled<T>(Gt + 16 * ct * L::LDT, L::LDT, lane, isc[0])));
                mma_xs<T>(Sacc[pi][ct], qb, split8<T>(ld8_scaled<T>(Gt + 16 * ct * L::LDT + 32, L::LDT, lane, isc[1])));
                if (b > 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) Sf[(p0 + 4 * g + i) * L::LDSF + 16 * ct + r] = Sacc[pi][ct][i];
                }
            }
            floatx4 zacc = zero4();
            mma_xs<T>(zacc, qa, dd0);
            mma_xs<T>(zacc, qb, dd1);
            if (r == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) zs[p0 + 4 * g + i] += zacc[i];
            }
        }
        sh_zero = false;
    }
    float *dSg = dS_in + (size_t)grp * D * D;
#pragma unroll
    for (int pi = 0; pi < NPT; ++pi)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dSg[(size_t)(16 * (w + 4 * pi) + 4 * g + i) * D + 16 * ct + r] = Sacc[pi][ct][i];
    __syncthreads();
    if (tid < D) dz_in[(size_t)grp * D + tid] = zs[tid];
}

template <typename T, int D>
hipError_t launch_bwd(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                      const void *dO, const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv,
                      float *dS_in, float *dz_in, int G, int C, hipStream_t stream) {
    hipLaunchKernelGGL((la_bwd_kernel<T, D>), dim3((unsigned)G), dim3(NTHR), 0, stream,
                       (const T *)q, (const T *)k, (const T *)v, S_in, z_in, (const T *)dO, dS_out, dz_out,
                       (T *)dq, (T *)dk, (T *)dv, dS_in, dz_in, C);
    return hipGetLastError();
}

template hipError_t launch_bwd<float, 64>(const void *, const void *, const void *, const float *, const float *,
                                          const void *, const float *, const float *, void *, void *, void *,
                                          float *, float *, int, int, hipStream_t);
template hipError_t launch_bwd<bf16, 64>(const void *, const void *, const void *, const float *, const float *,
                                         const void *, const float *, const float *, void *, void *, void *,
                                         float *, float *, int, int, hipStream_t);
template hipError_t launch_bwd<bf16, 128>(const void *, const void *, const void *, const float *, const float *,
                                          const void *, const float *, const float *, void *, void *, void *,
                                          float *, float *, int, int, hipStream_t);

}  // namespace lachunk
