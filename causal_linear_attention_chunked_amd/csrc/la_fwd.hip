// Forward kernel: one chunk of causal linear attention with a carried state,
// blocked form ("Fractus-1B training optimization", section 2, Opt 2) with the
// exact per-token cumsum for the ragged tail.
//
// Grid: one workgroup per (group, 64-wide slice of value columns); 8 waves, two per SIMD.
// The 64-token blocks are taken WIN at a time (a window; WIN = 2 except fp32 at D = 128).
// Only the running state carries a dependency from one block to the next, and it
// is cheap, so inside a window the state is advanced first and the blocks'
// outputs are then computed side by side, waves 0-3 on the first block, 4-7 on
// the second.  Per block b of a window, with S_b / z_b the state before it:
//   S_b+1   = S_b + K_b^T V_b,   z_b+1 = z_b + K_b^T 1                [update]
//   P^T     = K_b Q_b^T, masked to j <= t (inclusive)                 [wave: 16 queries]
//   num^T   = V_b^T P^T + S_b^T Q_b^T                                  [all 64 value columns]
//   den     = 1^T P^T + z_b^T Q_b^T                                    [a ones row: no shuffles]
//   o_t     = num_t / den_t
// then the ragged tail token by token: S += k v^T, z += k, o = S^T q / (q . z).
// The state lives in the waves' MFMA accumulators (fp32) and, for operand reads,
// as a bf16 S^T copy per block start in LDS.  The intra-block scores P enter the
// MFMAs as split hi + lo operands; the state copy does not need to (its term
// has no cancellation against the others).  Staging is natural row-major only:
// transposed operands come from LDS transpose reads.  The next window's loads
// are issued as soon as the current window is staged.
#include "la_common.h"
#include "la_launch.h"
#include <hip/hip_ext.h>

namespace lachunk {

template <typename T, int D> constexpr int fwd_window() { return (is_bf16<T>() || D == 64) ? 2 : 1; }

template <typename T, int D>
struct FwdLds {
    static constexpr int WIN = fwd_window<T, D>();
    static constexpr int PAD = Elem<T>::PAD;
    static constexpr int LDN = D + PAD;    // K rows [WIN*BK][LDN]
    // V slice rows [WIN*BK][LDV]: read only through transposed fragment reads, which are free of
    // bank conflicts at a 40-dword row pitch for bf16
    static constexpr int LDV = is_bf16<T>() ? 64 + 16 : 64 + PAD;
    static constexpr int LDST = D + PAD;   // S^T copies [64 value columns][LDST]
    static constexpr int LDSF = 64 + 4;    // fp32 state, tail phase
    static constexpr int ESZ = (int)sizeof(T);
    static constexpr int ZS = 0;                                   // [WIN][D] z at the block starts
    static constexpr int ST = ZS + WIN * D * 4;                    // [WIN][64][LDST]
    static constexpr int ST_ELEMS = 64 * LDST;
    static constexpr int KB = ST + WIN * ST_ELEMS * ESZ;            // [WIN*BK][LDN]
    static constexpr int VB = KB + WIN * BK * LDN * ESZ;            // [WIN*BK][LDV]
    static constexpr int TQ = VB + WIN * BK * LDV * ESZ;            // tail queries [BK][LDN]
    static constexpr int SF = TQ + BK * LDN * ESZ;                  // tail state [D][LDSF] fp32
    static constexpr int BYTES = SF + D * LDSF * 4;
    static_assert(ST % 16 == 0 && KB % 16 == 0 && VB % 16 == 0 && TQ % 16 == 0 && SF % 16 == 0, "LDS alignment");
    static_assert(BYTES <= 160 * 1024, "forward LDS budget exceeded");
};

// fp32 values z[kslot(lane, s)] of one k-chunk, the same for every row of the fragment
__device__ __forceinline__ floatx8 zrow8(const float *z, int lane) {
    const float *p = z + 4 * (lane >> 4);
    const floatx4 a = *reinterpret_cast<const floatx4 *>(p);
    const floatx4 b = *reinterpret_cast<const floatx4 *>(p + 16);
    return floatx8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <typename T, int D>
__global__ __launch_bounds__(NTHR, 1) void la_fwd_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in,
    T *__restrict__ o, float *__restrict__ S_out, float *__restrict__ z_out, int C) {
    using L = FwdLds<T, D>;
    constexpr int WIN = L::WIN;
    constexpr int NVS = D / 64;          // value slices per group
    constexpr int NKC = D / 32;          // k-chunks over the feature dimension
    constexpr int NOWN = D / 32;         // state tiles per wave (16 x 16 each)
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    float *zs = reinterpret_cast<float *>(smem + L::ZS);
    T *ST = reinterpret_cast<T *>(smem + L::ST);
    T *Ks = reinterpret_cast<T *>(smem + L::KB);
    T *Vs = reinterpret_cast<T *>(smem + L::VB);

    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (scalar)
    // outputs: block `blk` of the window, query tile tq (reversed on the second block, so
    // waves that share a SIMD carry one long and one short causal row range)
    const int blk = w >> 2;
    const int tq = blk ? 3 - (w & 3) : (w & 3);
    // state: value tile ct, key-feature tiles pt0 + 2i
    const int ct = w & 3, pt0 = w >> 2;
    const int grp = blockIdx.x / NVS, vs = blockIdx.x % NVS;
    const size_t tok0 = (size_t)grp * C;
    const uint32_t chunk_bytes = (uint32_t)C * D * sizeof(T);
    const GRes qr(q + tok0 * D, chunk_bytes), kr(k + tok0 * D, chunk_bytes), vr(v + tok0 * D, chunk_bytes);
    // an absent carry is an empty range (reads give zero); the base only has to be a valid address
    const GRes sres(S_in ? (const void *)(S_in + (size_t)grp * D * D) : (const void *)S_out, S_in ? D * D * 4 : 0);
    const GRes zres(z_in ? (const void *)(z_in + (size_t)grp * D) : (const void *)z_out, z_in ? D * 4 : 0);
    // waves without a block of their own (one-block windows) read nothing
    const GRes qw(q + tok0 * D, blk < WIN ? chunk_bytes : 0);
    T *og = o + tok0 * D + vs * 64;
    const int nb = C / BK, tail = C % BK;
    const int nwin = (nb + WIN - 1) / WIN;

    struct Window {
        Stager<T, D> k[WIN];
        Stager<T, 64> v[WIN];
        Frag<T> qf[NKC];
    };
    auto load_window = [&](Window &x, int wi) {  // rows past the chunk read as zero
        const uint32_t t0 = (uint32_t)wi * WIN * BK;
#pragma unroll
        for (int bi = 0; bi < WIN; ++bi) {
            x.k[bi].load(kr, (t0 + bi * BK) * D, D, tid);
            x.v[bi].load(vr, (t0 + bi * BK) * D + vs * 64, D, tid);
        }
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
            x.qf[kc] = ldfrag_g<T>(qw, (t0 + blk * BK + 16 * tq) * D + 32 * kc, D, lane);
    };
    auto store_window = [&](const Window &x) {
#pragma unroll
        for (int bi = 0; bi < WIN; ++bi) {
            x.k[bi].store(Ks + bi * BK * L::LDN, L::LDN, nullptr, 0, tid);
            x.v[bi].store(Vs + bi * BK * L::LDV, L::LDV, nullptr, 0, tid);
        }
    };

    // ---- prologue: window 0, the tail's queries and the carry, all issued before any wait
    Window nxt;
    load_window(nxt, 0);
    Stager<T, D> qtail;
    qtail.load(tail ? qr : GRes(q, 0), (uint32_t)nb * BK * D, D, tid);
    floatx4 Sacc[NOWN];  // S[p][c], p-tile pt0 + 2i, c-tile ct: lane (c = r), element e: p = 4g + e
    floatx4 zr[NOWN];    // z[p] for the same p-tiles (every lane; kept current by the waves of c-tile 0)
#pragma unroll
    for (int i = 0; i < NOWN; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int p = 16 * (pt0 + 2 * i) + 4 * g + e;
            Sacc[i][e] = gload<float>(sres, (p * D + vs * 64 + 16 * ct + r) * 4);
            zr[i][e] = gload<float>(zres, p * 4);
        }
    __syncthreads();  // keeps every prologue load issued here, ahead of the first wait

    // state copy s <- (Sacc, zr); z is written by the waves of value tile 0
    auto write_state = [&](int s) {
#pragma unroll
        for (int i = 0; i < NOWN; ++i) {
            const int p0 = 16 * (pt0 + 2 * i) + 4 * g;
            *reinterpret_cast<Vec4<T> *>(ST + s * L::ST_ELEMS + (16 * ct + r) * L::LDST + p0) = to_vec4<T>(Sacc[i]);
            if (ct == 0 && r == 0) *reinterpret_cast<floatx4 *>(zs + s * D + p0) = zr[i];
        }
    };
    const Frag<T> ones = ones_frag<T>();
    // S += K_bi^T V_bi and z += K_bi^T 1 over one staged block
    auto update = [&](int bi) {
#pragma unroll
        for (int kc2 = 0; kc2 < 2; ++kc2) {
            const int t0 = bi * BK + 32 * kc2;
            const Frag<T> vt = ldfrag_tr<T>(Vs + t0 * L::LDV + 16 * ct, L::LDV, lane);
#pragma unroll
            for (int i = 0; i < NOWN; ++i) {
                const Frag<T> kt = ldfrag_tr<T>(Ks + t0 * L::LDN + 16 * (pt0 + 2 * i), L::LDN, lane);
                mma(Sacc[i], kt, vt);
                if (ct == 0) mma(zr[i], kt, ones);
            }
        }
    };
    write_state(0);

    for (int wi = 0; wi < nwin; ++wi) {
        const int nblk = (nb - wi * WIN) < WIN ? (nb - wi * WIN) : WIN;
        const int t0 = wi * WIN * BK;
        store_window(nxt);
        Frag<T> qc[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) qc[kc] = nxt.qf[kc];
        // the next window, or the blocks after the last one when the ragged tail needs its keys and
        // values from them (reads past the chunk give zeros); nothing when neither is wanted, so the
        // barrier below does not wait on useless loads
        if (wi + 1 < nwin || (tail && nb % WIN == 0)) load_window(nxt, wi + 1);
        __syncthreads();           // window staged; state copy 0 visible

        if constexpr (WIN == 2) {  // state after the window's first block: copy 1
            update(0);
            write_state(1);
        }
        // intra-block part of this wave's outputs: needs only the staged K, V and its queries
        const bool active = blk < nblk;
        const T *Kb = Ks + blk * BK * L::LDN;
        const T *Vb = Vs + blk * BK * L::LDV;
        floatx4 nm[4], dn = zero4();
#pragma unroll
        for (int c = 0; c < 4; ++c) nm[c] = zero4();
        if (active) {
            floatx4 sc[4];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                sc[jt] = zero4();
                if (jt <= tq) {
#pragma unroll
                    for (int kc = 0; kc < NKC; ++kc)
                        mma(sc[jt], ldfrag<T>(Kb + 16 * jt * L::LDN + 32 * kc, L::LDN, lane), qc[kc]);
                }
                if (jt == tq) {  // diagonal tile: keep key j <= query t
#pragma unroll
                    for (int e = 0; e < 4; ++e) sc[jt][e] = 4 * g + e <= r ? sc[jt][e] : 0.f;
                }
            }
            const SFrag<T> pf0 = split8<T>(acc8(sc[0], sc[1]));
            mma_xs<T>(dn, ones, pf0);
#pragma unroll
            for (int c = 0; c < 4; ++c) mma_xs<T>(nm[c], ldfrag_tr<T>(Vb + 16 * c, L::LDV, lane), pf0);
            if (tq >= 2) {
                const SFrag<T> pf1 = split8<T>(acc8(sc[2], sc[3]));
                mma_xs<T>(dn, ones, pf1);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    mma_xs<T>(nm[c], ldfrag_tr<T>(Vb + 32 * L::LDV + 16 * c, L::LDV, lane), pf1);
            }
        }
        if constexpr (WIN == 2) __syncthreads();  // state copy 1 visible
        if (active) {
            // inter-block part: the state before this block, read before it is updated
            const T *STb = ST + blk * L::ST_ELEMS;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                mma_sx<T>(dn, split8<T>(zrow8(zs + blk * D + 32 * kc, lane)), qc[kc]);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    mma(nm[c], ldfrag<T>(STb + 16 * c * L::LDST + 32 * kc, L::LDST, lane), qc[kc]);
            }
            const float inv = __builtin_amdgcn_rcpf(dn[0]);
            T *orow = og + (size_t)(t0 + blk * BK + 16 * tq + r) * D + 4 * g;
#pragma unroll
            for (int c = 0; c < 4; ++c) *reinterpret_cast<Vec4<T> *>(orow + 16 * c) = to_vec4<T>(nm[c] * inv);
        }
        // state after the window
        if constexpr (WIN == 2) {
            if (nblk == 2) update(1);
        } else {
            update(0);
        }
        if (wi + 1 < nwin) {
            __syncthreads();  // every wave is done reading this window's staging and state copies
            write_state(0);
        }
    }

    if (tail == 0) {
        float *Sg = S_out + (size_t)grp * D * D + vs * 64 + 16 * ct + r;
#pragma unroll
        for (int i = 0; i < NOWN; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) Sg[(size_t)(16 * (pt0 + 2 * i) + 4 * g + e) * D] = Sacc[i][e];
        if (vs == 0 && ct == 0 && r == 0) {
#pragma unroll
            for (int i = 0; i < NOWN; ++i)
                *reinterpret_cast<floatx4 *>(z_out + (size_t)grp * D + 16 * (pt0 + 2 * i) + 4 * g) = zr[i];
        }
        return;
    }

    // ---- ragged tail: exact per-token cumsum from (S_run, z_run).  Its keys and values are
    // either the empty block slot of the last window (already staged) or the prefetch of the
    // window after it (still in registers).
    T *Tq = reinterpret_cast<T *>(smem + L::TQ);
    float *Sf = reinterpret_cast<float *>(smem + L::SF);
    const int slot = nb % WIN;
    const int tt0 = nb * BK;
    if (nwin > 0) __syncthreads();  // the window phase is finished with the staging space
    if (slot == 0) {
        nxt.k[0].store(Ks, L::LDN, nullptr, 0, tid);
        nxt.v[0].store(Vs, L::LDV, nullptr, 0, tid);
    }
    qtail.store(Tq, L::LDN, nullptr, 0, tid);
#pragma unroll
    for (int i = 0; i < NOWN; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int p = 16 * (pt0 + 2 * i) + 4 * g + e;
            Sf[p * L::LDSF + 16 * ct + r] = Sacc[i][e];
            if (ct == 0 && r == 0) zs[p] = zr[i][e];
        }
    __syncthreads();
    if (w >= 4) return;  // no barrier follows
    const T *Tk = Ks + slot * BK * L::LDN;
    const T *Tv = Vs + slot * BK * L::LDV;
    // lane owns value column c = 16w + r of the slice and key features p in [g*NP, (g+1)*NP)
    constexpr int NP = D / 4;
    const int c = 16 * w + r;
    float Sr[NP], zl[NP];
#pragma unroll
    for (int s = 0; s < NP; ++s) {
        Sr[s] = Sf[(g * NP + s) * L::LDSF + c];
        zl[s] = zs[g * NP + s];
    }
    for (int t = 0; t < tail; ++t) {
        const float vc = tof(Tv[t * L::LDV + c]);
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
                zl[s4 + e] += kp;
                n += qp * Sr[s4 + e];
                d += qp * zl[s4 + e];
            }
        }
        n = wsum_g(n);
        d = wsum_g(d);
        if (g == 0) og[(size_t)(tt0 + t) * D + c] = fromf<T>(n / d);
    }
    float *Sg = S_out + (size_t)grp * D * D + vs * 64;
#pragma unroll
    for (int s = 0; s < NP; ++s) Sg[(size_t)(g * NP + s) * D + c] = Sr[s];
    if (vs == 0 && w == 0 && r == 0) {
#pragma unroll
        for (int s = 0; s < NP; ++s) z_out[(size_t)grp * D + g * NP + s] = zl[s];
    }
}

template <typename T, int D>
hipError_t launch_fwd(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                      void *o, float *S_out, float *z_out, int G, int C, hipStream_t stream,
                      const hipEvent_t ev[2]) {
    dim3 grid((unsigned)G * (D / 64)), block(NTHR);
    hipExtLaunchKernelGGL((la_fwd_kernel<T, D>), grid, block, 0, stream, ev[0], ev[1], 0,
                          (const T *)q, (const T *)k, (const T *)v, S_in, z_in, (T *)o, S_out, z_out, C);
    return hipGetLastError();
}

template hipError_t launch_fwd<float, 64>(const void *, const void *, const void *, const float *, const float *,
                                          void *, float *, float *, int, int, hipStream_t, const hipEvent_t *);
template hipError_t launch_fwd<float, 128>(const void *, const void *, const void *, const float *, const float *,
                                           void *, float *, float *, int, int, hipStream_t, const hipEvent_t *);
template hipError_t launch_fwd<bf16, 64>(const void *, const void *, const void *, const float *, const float *,
                                         void *, float *, float *, int, int, hipStream_t, const hipEvent_t *);
template hipError_t launch_fwd<bf16, 128>(const void *, const void *, const void *, const float *, const float *,
                                          void *, float *, float *, int, int, hipStream_t, const hipEvent_t *);

}  // namespace lachunk
