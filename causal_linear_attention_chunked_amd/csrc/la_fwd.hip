// Forward kernel: one chunk of causal linear attention with a carried state,
// blocked form ("Fractus-1B training optimization", section 2, Opt 2) with the
// exact per-token cumsum for the ragged tail.
//
// Grid: one workgroup per (group, 64-wide slice of value columns); 8 waves, two per SIMD.
// Per 64-token block b, with the running state S_run (fp32 MFMA accumulators
// spread over the waves, mirrored in LDS as split S^T copies) and z_run (LDS):
//   scores  P^T = K_b Q_b^T, masked to j <= t (inclusive)   [wave w: queries 16w..16w+15]
//   den_t   = sum_j P[t][j] + q_t . z_run                     [row sums by lane shuffles]
//   num^T   = V_b^T P^T + S_run^T Q_b^T                       [state read BEFORE the update]
//   o_t     = num_t / den_t
//   S_run  += K_b^T V_b,  z_run += K_b^T 1                    [update after reading]
// then the ragged tail token by token: S += k v^T, z += k, o = S^T q / (q . z).
// Staging is natural row-major only: transposed operands (K^T, V^T) come from
// LDS transpose reads.  Blocks are double-buffered in LDS and loaded two ahead.
#include "la_common.h"
#include "la_launch.h"

namespace lachunk {

template <typename T, int D>
struct FwdLds {
    static constexpr int PAD = Elem<T>::PAD;
    static constexpr int LDN = D + PAD;    // K rows [BK][LDN]
    static constexpr int LDV = 64 + PAD;   // V slice rows [BK][LDV]
    static constexpr int LDST = D + PAD;   // S^T copies [64 value columns][LDST]
    static constexpr int NCOPY = is_bf16<T>() ? 2 : 1;
    static constexpr int ZS = 0;                                         // [NTHR] z_run (first D used)
    static constexpr int STH = NTHR * 4;                                 // S^T hi
    static constexpr int STL = STH + 64 * LDST * (int)sizeof(T);         // S^T lo (bf16 only)
    static constexpr int STAGE = STH + NCOPY * 64 * LDST * (int)sizeof(T);
    static constexpr int KBUF = BK * LDN * (int)sizeof(T);
    static constexpr int VBUF = BK * LDV * (int)sizeof(T);
    static constexpr int BLOCK_END = STAGE + 2 * (KBUF + VBUF);          // two staging buffers
    // ragged-tail phase (reuses the staging space)
    static constexpr int LDSF = 64 + 4;
    static constexpr int TQ = STAGE, TK = TQ + KBUF, TV = TK + KBUF, SF = TV + VBUF;
    static constexpr int TAIL_END = SF + D * LDSF * 4;
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
    constexpr int NPT = D / 64;          // key-feature tiles of the state per wave
    constexpr int NKC = D / 32;          // k-chunks over the feature dimension
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    float *zs = reinterpret_cast<float *>(smem + L::ZS);
    T *STh = reinterpret_cast<T *>(smem + L::STH);
    T *STl = reinterpret_cast<T *>(smem + L::STL);
    auto Kbuf = [&](int i) { return reinterpret_cast<T *>(smem + L::STAGE + i * (L::KBUF + L::VBUF)); };
    auto Vbuf = [&](int i) { return reinterpret_cast<T *>(smem + L::STAGE + i * (L::KBUF + L::VBUF) + L::KBUF); };

    // wave w: query tile tq = w % 4 (16 tokens of each block) and value-column half hh = w / 4
    // (column tiles 2hh, 2hh+1 of the 64-wide slice); the same pair indexes its share of the state
    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (scalar)
    const int tq = w & 3, hh = w >> 2;
    const int grp = blockIdx.x / NVS, vs = blockIdx.x % NVS;
    const size_t tok0 = (size_t)grp * C;
    const uint32_t chunk_bytes = (uint32_t)C * D * sizeof(T);
    const GRes qr(q + tok0 * D, chunk_bytes), kr(k + tok0 * D, chunk_bytes), vr(v + tok0 * D, chunk_bytes);
    // an absent carry is an empty range (reads give zero); the base only has to be a valid address
    const GRes sres(S_in ? (const void *)(S_in + (size_t)grp * D * D) : (const void *)S_out, S_in ? D * D * 4 : 0);
    const GRes zres(z_in ? (const void *)(z_in + (size_t)grp * D) : (const void *)z_out, z_in ? D * 4 : 0);
    T *og = o + tok0 * D + vs * 64;
    const int nb = C / BK, tail = C % BK;

    struct Block {
        Stager<T, D> k;
        Stager<T, 64> v;
        Frag<T> qf[NKC];
    };
    auto load_block = [&](Block &x, int b) {  // blocks past the chunk read as zero
        const uint32_t t0 = (uint32_t)b * BK;
        x.k.load(kr, t0 * D, D, tid);
        x.v.load(vr, t0 * D + vs * 64, D, tid);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) x.qf[kc] = ldfrag_g<T>(qr, (t0 + 16 * tq) * D + 32 * kc, D, lane);
    };
    auto store_block = [&](const Block &x, int buf) {
        x.k.store(Kbuf(buf), L::LDN, nullptr, 0, tid);
        x.v.store(Vbuf(buf), L::LDV, nullptr, 0, tid);
    };

    // ---- prologue: block 0 and the carry.  Each loop iteration first moves the block
    // prefetched into registers to its LDS buffer and at once issues the next block's loads,
    // which then run under this block's compute.
    Block nxt;
    load_block(nxt, 0);
    floatx4 Sacc[NPT][2];  // acc(p, c): p-tiles tq + 4*pi, c-tiles 2hh + cc
#pragma unroll
    for (int pi = 0; pi < NPT; ++pi)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Sacc[pi][cc][i] = gload<float>(sres, ((16 * (tq + 4 * pi) + 4 * g + i) * D + vs * 64 + 16 * (2 * hh + cc) + r) * 4);
    const float zin = gload<float>(zres, tid * 4);  // threads past D read zero
    __syncthreads();  // keeps every prologue load issued here, ahead of the first wait
    auto write_copies = [&]() {
#pragma unroll
        for (int pi = 0; pi < NPT; ++pi)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int off = (16 * (2 * hh + cc) + r) * L::LDST + 16 * (tq + 4 * pi) + 4 * g;
                store_split4<T>(STh + off, STl + off, Sacc[pi][cc]);
            }
    };
    write_copies();
    zs[tid] = zin;

    const Frag<T> ones = ones_frag<T>();
    for (int b = 0; b < nb; ++b) {
        const int t0 = b * BK, buf = b & 1;
        const T *Kn = Kbuf(buf), *Vn = Vbuf(buf);
        store_block(nxt, buf);
        Frag<T> qc[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) qc[kc] = nxt.qf[kc];
        load_block(nxt, b + 1);  // past the end of the chunk: zeros, no memory traffic
        __syncthreads();  // block b staged; the previous update of the state copies and z_run visible
        // scores P^T[j][t] for every key tile (tiles after the diagonal are masked to zero)
        floatx4 sc[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) sc[jt] = zero4();
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            Frag<T> kf[4];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) kf[jt] = ldfrag<T>(Kn + 16 * jt * L::LDN + 32 * kc, L::LDN, lane);
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) mma(sc[jt], kf[jt], qc[kc]);
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool keep = jt < tq || (jt == tq && 4 * g + i <= r);
                sc[jt][i] = keep ? sc[jt][i] : 0.f;
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

        // num^T[c][t] = V^T P^T (intra) + S_run^T Q^T (inter, state before this block), own columns
        Frag<T> vt[2][2];  // V^T rows c (k = key), reused by the state update
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int h = 0; h < 2; ++h) vt[cc][h] = ldfrag_tr<T>(Vn + 32 * h * L::LDV + 16 * (2 * hh + cc), L::LDV, lane);
        {
            const SFrag<T> pf0 = split8<T>(acc8(sc[0], sc[1]));
            const SFrag<T> pf1 = split8<T>(acc8(sc[2], sc[3]));
            floatx4 nm[2];
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                nm[cc] = zero4();
                mma_xs<T>(nm[cc], vt[cc][0], pf0);
                mma_xs<T>(nm[cc], vt[cc][1], pf1);
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) {
                    const int off = 16 * (2 * hh + cc) * L::LDST + 32 * kc;
                    mma_sx<T>(nm[cc], ldsplit<T>(STh + off, STl + off, L::LDST, lane), qc[kc]);
                }
            }
            T *orow = og + (size_t)(t0 + 16 * tq + r) * D + 32 * hh + 4 * g;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) *reinterpret_cast<Vec4<T> *>(orow + 16 * cc) = to_vec4<T>(nm[cc] * inv);
        }
        __syncthreads();  // every wave is done reading the state copies and z_run of this block

        // update after reading: S_run += K^T V, z_run += K^T 1
#pragma unroll
        for (int pi = 0; pi < NPT; ++pi) {
            const int p0 = 16 * (tq + 4 * pi);
            const Frag<T> kt0 = ldfrag_tr<T>(Kn + p0, L::LDN, lane);
            const Frag<T> kt1 = ldfrag_tr<T>(Kn + 32 * L::LDN + p0, L::LDN, lane);
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                mma(Sacc[pi][cc], kt0, vt[cc][0]);
                mma(Sacc[pi][cc], kt1, vt[cc][1]);
            }
            if (hh == 0) {
                floatx4 zacc = zero4();
                mma(zacc, kt0, ones);
                mma(zacc, kt1, ones);
                if (r == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) zs[p0 + 4 * g + i] += zacc[i];
                }
            }
        }
        write_copies();
    }

    if (tail == 0) {
        float *Sg = S_out + (size_t)grp * D * D + vs * 64;
#pragma unroll
        for (int pi = 0; pi < NPT; ++pi)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Sg[(size_t)(16 * (tq + 4 * pi) + 4 * g + i) * D + 16 * (2 * hh + cc) + r] = Sacc[pi][cc][i];
        __syncthreads();
        if (vs == 0 && tid < D) z_out[(size_t)grp * D + tid] = zs[tid];
        return;
    }

    // ---- ragged tail: exact per-token cumsum from (S_run, z_run); waves 0..3 own the columns
    T *Tq = reinterpret_cast<T *>(smem + L::TQ);
    T *Tk = reinterpret_cast<T *>(smem + L::TK);
    T *Tv = reinterpret_cast<T *>(smem + L::TV);
    float *Sf = reinterpret_cast<float *>(smem + L::SF);
    const int tt0 = nb * BK;
    {
        Stager<T, D> qs, ks;
        Stager<T, 64> vs_;
        qs.load(qr, tt0 * D, D, tid);  // rows past the chunk read as zero
        ks.load(kr, tt0 * D, D, tid);
        vs_.load(vr, tt0 * D + vs * 64, D, tid);
        __syncthreads();  // the block phase is finished with the staging space
#pragma unroll
        for (int pi = 0; pi < NPT; ++pi)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Sf[(16 * (tq + 4 * pi) + 4 * g + i) * L::LDSF + 16 * (2 * hh + cc) + r] = Sacc[pi][cc][i];
        qs.store(Tq, L::LDN, nullptr, 0, tid);
        ks.store(Tk, L::LDN, nullptr, 0, tid);
        vs_.store(Tv, L::LDV, nullptr, 0, tid);
        __syncthreads();
    }
    if (w >= 4) return;  // no barrier follows
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
                zr[s4 + e] += kp;
                n += qp * Sr[s4 + e];
                d += qp * zr[s4 + e];
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
