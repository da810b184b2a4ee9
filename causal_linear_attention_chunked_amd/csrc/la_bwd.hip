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
// Grid: one workgroup per group, 8 waves (two per SIMD).  Every fp32 intermediate (P, dP, dN,
// dden, S, Sh) enters the MFMAs as a bf16 hi + lo pair (see la_common.h).  The
// state lives in the waves' accumulators and, for operand reads, as split S^T
// copies in LDS read directly (S^T) or through transpose reads (S).  Staging
// holds natural row-major tiles only, double-buffered and loaded two blocks ahead.
#include "la_common.h"
#include "la_launch.h"
#include <hip/hip_ext.h>
#include "../../include/la_chunk.h"

namespace lachunk {

template <typename T, int D>
struct BwdLds {
    static constexpr int PAD = Elem<T>::PAD;
    static constexpr int LDN = D + PAD;    // token-major tiles [BK][LDN]
    static constexpr int LDST = D + PAD;   // state copies S^T[c][p]
    static constexpr int LDSF = D + 4;     // fp32 state in the tail phase
    static constexpr int NCOPY = is_bf16<T>() ? 2 : 1;
    static constexpr int NBUF = D <= 64 ? 2 : 1;   // staging buffers (one at D = 128: LDS)
    static constexpr int CMAX = LA_BWD_MAX_C;
    static constexpr int ZS = 0;                                  // [D] z_b (pass 1) / zh (pass 2)
    static constexpr int DEN = ZS + D * 4;                        // [CMAX] den_t
    static constexpr int DDEN = DEN + CMAX * 4;                   // [CMAX] dden_t
    static constexpr int XROW = DDEN + CMAX * 4;                  // [2][BK] row-dot halves
    static constexpr int PART = XROW + 2 * BK * 4;                // [2][NWAVE] tail row-dot partials
    static constexpr int STH = ((PART + 2 * NWAVE * 4 + 15) / 16) * 16;
    static constexpr int STL = STH + D * LDST * (int)sizeof(T);
    static constexpr int SF = STH;                                // fp32 state, tail phase only
    static constexpr int WORK = STH + NCOPY * D * LDST * (int)sizeof(T);
    static constexpr int TILE = BK * LDN * (int)sizeof(T);
    // pass 1: NBUF x {K, V} staging, then the exchanged dN (hi, lo)
    static constexpr int P1_STAGE = WORK, DNX = WORK + NBUF * 2 * TILE;
    static constexpr int P1_END = DNX + 2 * TILE;
    // pass 2: NBUF x {Q, dN hi, dN lo}
    static constexpr int P2_STAGE = WORK, P2_END = WORK + NBUF * 3 * TILE;
    // tail: q, k, v, dO rows
    static constexpr int TAIL_END = WORK + 4 * TILE;
    static constexpr int BYTES = P1_END > P2_END ? (P1_END > TAIL_END ? P1_END : TAIL_END)
                                                 : (P2_END > TAIL_END ? P2_END : TAIL_END);
    static_assert(D * LDSF * 4 <= NCOPY * D * LDST * (int)sizeof(T), "tail state does not fit the copies");
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
    constexpr int NPT = D / 64;          // state row tiles per wave
    constexpr int NCT = D / 16;          // feature tiles
    constexpr int NHT = NCT / 2;         // feature tiles of one half
    constexpr int NKC = D / 32;          // k-chunks over the feature dimension
    constexpr bool TWOBUF = L::NBUF == 2;  // two staging buffers (one at D = 128)
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    float *zs = reinterpret_cast<float *>(smem + L::ZS);
    float *den_all = reinterpret_cast<float *>(smem + L::DEN);
    float *dden_all = reinterpret_cast<float *>(smem + L::DDEN);
    float *xrow = reinterpret_cast<float *>(smem + L::XROW);
    float *part = reinterpret_cast<float *>(smem + L::PART);
    float *Sf = reinterpret_cast<float *>(smem + L::SF);
    T *STh = reinterpret_cast<T *>(smem + L::STH);
    T *STl = reinterpret_cast<T *>(smem + L::STL);
    T *DNh = reinterpret_cast<T *>(smem + L::DNX);
    T *DNl = reinterpret_cast<T *>(smem + L::DNX + L::TILE);
    auto tile1 = [&](int buf, int which) { return reinterpret_cast<T *>(smem + L::P1_STAGE + (2 * buf + which) * L::TILE); };
    auto tile2 = [&](int buf, int which) { return reinterpret_cast<T *>(smem + L::P2_STAGE + (3 * buf + which) * L::TILE); };

    // wave w: token tile tq = w % 4 (queries in pass 1, keys in pass 2) and half hh = w / 4
    // (feature half in pass 1 and in the state updates; in pass 2 half 0 forms dV, half 1 dK)
    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (scalar)
    const int tq = w & 3, hh = w >> 2;
    const int grp = blockIdx.x;
    const size_t tok0 = (size_t)grp * C;
    const uint32_t chunk_bytes = (uint32_t)C * D * sizeof(T);
    const GRes qres(q + tok0 * D, chunk_bytes), kres(k + tok0 * D, chunk_bytes), vres(v + tok0 * D, chunk_bytes),
        gres(dO + tok0 * D, chunk_bytes);
    const GRes none(dq, 0);  // an empty range: every read gives zero
    T *dqg = dq + tok0 * D, *dkg = dk + tok0 * D, *dvg = dv + tok0 * D;
    const int nb = C / BK, tail = C % BK, tt0 = nb * BK;
    const int past = nb + 2;  // a block index whose rows all lie past the chunk
    const Frag<T> ones = ones_frag<T>();

    floatx4 Sacc[NPT][NHT];  // state acc(p, c): p-tiles tq + 4*pi, c-tiles hh*NHT + cc
    auto ptile = [&](int pi) { return 16 * (tq + 4 * pi); };
    auto ctile = [&](int cc) { return 16 * (hh * NHT + cc); };
    auto write_copies = [&]() {
#pragma unroll
        for (int pi = 0; pi < NPT; ++pi)
#pragma unroll
            for (int cc = 0; cc < NHT; ++cc) {
                const int off = (ctile(cc) + r) * L::LDST + ptile(pi) + 4 * g;
                store_split4<T>(STh + off, STl + off, Sacc[pi][cc]);
            }
    };
    auto load_state = [&](const GRes &src) {  // [D][D] fp32; an empty range gives zeros
#pragma unroll
        for (int pi = 0; pi < NPT; ++pi)
#pragma unroll
            for (int cc = 0; cc < NHT; ++cc)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Sacc[pi][cc][i] = gload<float>(src, ((ptile(pi) + 4 * g + i) * D + ctile(cc) + r) * 4);
    };

    // One block's loads.  Pass 1 stages K and V and keeps this wave's Q rows (f) and this half's
    // dO columns (gv) in registers; pass 2 stages Q and dO and keeps this wave's K rows (half 0)
    // or V rows (half 1).  The pass is a uniform flag, so the sources are scalar selects.
    struct Block {
        Stager<T, D> a, b;
        Frag<T> f[NKC];
        Vec4<T> gv[NHT];
    };
    auto load_block = [&](Block &x, int blk, bool pass2) {
        const uint32_t t0 = (uint32_t)blk * BK, row = t0 + 16 * tq;
        const GRes ra = pass2 ? qres : kres, rb = pass2 ? gres : vres;
        const GRes rf = pass2 ? (hh == 0 ? kres : vres) : qres, rg = pass2 ? none : gres;
        x.a.load(ra, t0 * D, D, tid);
        x.b.load(rb, t0 * D, D, tid);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) x.f[kc] = ldfrag_g<T>(rf, row * D + 32 * kc, D, lane);
#pragma unroll
        for (int cc = 0; cc < NHT; ++cc) x.gv[cc] = gload<Vec4<T>>(rg, ((row + r) * D + ctile(cc) + 4 * g) * sizeof(T));
    };
    auto stage1 = [&](const Block &x, int buf) {
        x.a.store(tile1(buf, 0), L::LDN, nullptr, 0, tid);
        x.b.store(tile1(buf, 1), L::LDN, nullptr, 0, tid);
    };
    auto stage2 = [&](const Block &x, int buf, int blk) {  // dN = dO / den, stored split
        x.a.store(tile2(buf, 0), L::LDN, nullptr, 0, tid);
        x.b.store_scaled_split(tile2(buf, 1), tile2(buf, 2), L::LDN, den_all + blk * BK, tid);
    };

    // ---- pass 1 prologue: block 0 and the carry; the barrier keeps the loads issued up front
    Block nxt;
    load_block(nxt, 0, false);
    load_state(S_in ? GRes(S_in + (size_t)grp * D * D, D * D * 4) : none);
    const float zin = gload<float>(z_in ? GRes(z_in + (size_t)grp * D, D * 4) : none, tid * 4);
    __syncthreads();
    write_copies();
    if (tid < D) zs[tid] = zin;

    // =========================== pass 1: forward sweep ===========================
    for (int b = 0; b < nb; ++b) {
        const int t0 = b * BK, buf = TWOBUF ? (b & 1) : 0;
        const T *Kn = tile1(buf, 0), *Vn = tile1(buf, 1);
        const bool last = b + 1 == nb;
        if (!TWOBUF) __syncthreads();  // one buffer: the previous block's update is done with it
        stage1(nxt, buf);
        Frag<T> qc[NKC];
        Vec4<T> gc[NHT];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) qc[kc] = nxt.f[kc];
#pragma unroll
        for (int cc = 0; cc < NHT; ++cc) gc[cc] = nxt.gv[cc];
        // prefetch: the next block, or after the last one pass 2's first block (none when a tail follows)
        const bool to_pass2 = last && tail == 0;
        load_block(nxt, !last ? b + 1 : (tail == 0 ? nb - 1 : past), to_pass2);
        __syncthreads();  // block staged; previous state update visible

        const int trow = t0 + 16 * tq + r;
        // scores P^T[j][t] (lane: query t = 16tq + r, keys 4g+i of tile jt), masked inclusively
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

        // this half's columns of num^T; dN = dO / den goes to LDS (split), the row dot to xrow
        {
            const SFrag<T> pf0 = split8<T>(acc8(sc[0], sc[1]));
            const SFrag<T> pf1 = split8<T>(acc8(sc[2], sc[3]));
            float rowdot = 0.f;
#pragma unroll
            for (int cc = 0; cc < NHT; ++cc) {
                floatx4 nm = zero4();
                mma_xs<T>(nm, ldfrag_tr<T>(Vn + ctile(cc), L::LDN, lane), pf0);
                mma_xs<T>(nm, ldfrag_tr<T>(Vn + 32 * L::LDN + ctile(cc), L::LDN, lane), pf1);
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) {
                    const int off = ctile(cc) * L::LDST + 32 * kc;
                    mma_sx<T>(nm, ldsplit<T>(STh + off, STl + off, L::LDST, lane), qc[kc]);
                }
                floatx4 dn;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float gi = tof(gc[cc][i]);
                    rowdot += gi * nm[i];
                    dn[i] = gi * inv;
                }
                const int off = (16 * tq + r) * L::LDN + ctile(cc) + 4 * g;
                store_split4<T>(DNh + off, DNl + off, dn);
            }
            rowdot = wsum_g(rowdot);
            if (g == 0) xrow[hh * BK + 16 * tq + r] = rowdot;
        }
        __syncthreads();  // both halves' dN and row dots are visible
        const float dden = -(xrow[16 * tq + r] + xrow[BK + 16 * tq + r]) * inv * inv;
        if (hh == 0 && g == 0) {
            den_all[trow] = dsum;
            dden_all[trow] = dden;
        }
        // dN rows t = 16tq.. as split fragments over every feature chunk
        SFrag<T> dNs[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            const int off = 16 * tq * L::LDN + 32 * kc;
            dNs[kc] = ldsplit<T>(DNh + off, DNl + off, L::LDN, lane);
        }
        // dP^T[j][t] = sum_c V[j][c] dN[t][c] + dden_t, masked j <= t
        floatx4 dp[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) dp[jt] = zero4();
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            Frag<T> vn[4];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) vn[jt] = ldfrag<T>(Vn + 16 * jt * L::LDN + 32 * kc, L::LDN, lane);
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) mma_xs<T>(dp[jt], vn[jt], dNs[kc]);
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool keep = jt < tq || (jt == tq && 4 * g + i <= r);
                dp[jt][i] = keep ? dp[jt][i] + dden : 0.f;
            }
        // dQ^T[p][t] = K^T dP^T + S_b dN^T + z_b dden for this half's feature tiles
        {
            const SFrag<T> df0 = split8<T>(acc8(dp[0], dp[1]));
            const SFrag<T> df1 = split8<T>(acc8(dp[2], dp[3]));
            floatx4 a[NHT];
#pragma unroll
            for (int pt = 0; pt < NHT; ++pt) {
                a[pt] = zero4();
                mma_xs<T>(a[pt], ldfrag_tr<T>(Kn + ctile(pt), L::LDN, lane), df0);
                mma_xs<T>(a[pt], ldfrag_tr<T>(Kn + 32 * L::LDN + ctile(pt), L::LDN, lane), df1);
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) {
                    const int off = 32 * kc * L::LDST + ctile(pt);
                    mma_ss<T>(a[pt], ldsplit_tr<T>(STh + off, STl + off, L::LDST, lane), dNs[kc]);
                }
            }
            T *drow = dqg + (size_t)trow * D + 4 * g;
#pragma unroll
            for (int pt = 0; pt < NHT; ++pt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) a[pt][i] += dden * zs[ctile(pt) + 4 * g + i];
                *reinterpret_cast<Vec4<T> *>(drow + ctile(pt)) = to_vec4<T>(a[pt]);
            }
        }
        if (to_pass2) break;  // the state after the last block is not needed
        __syncthreads();  // every wave is done reading the state copies, z_b and dN
        // S_b += K^T V, z_b += K^T 1
#pragma unroll
        for (int pi = 0; pi < NPT; ++pi) {
            const int p0 = ptile(pi);
            const Frag<T> kt0 = ldfrag_tr<T>(Kn + p0, L::LDN, lane);
            const Frag<T> kt1 = ldfrag_tr<T>(Kn + 32 * L::LDN + p0, L::LDN, lane);
#pragma unroll
            for (int cc = 0; cc < NHT; ++cc) {
                mma(Sacc[pi][cc], kt0, ldfrag_tr<T>(Vn + ctile(cc), L::LDN, lane));
                mma(Sacc[pi][cc], kt1, ldfrag_tr<T>(Vn + 32 * L::LDN + ctile(cc), L::LDN, lane));
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

    // =========================== ragged tail (both passes) ===========================
    // Token by token; waves 0..D/16-1 hold the state in two layouts (one column / one row per
    // lane), the other waves only join the barriers.
    constexpr int NP = D / 4;     // features per lane-group
    constexpr int NH = 1;         // columns (layout A) / rows (layout B) per lane
    constexpr int TW = D / 16;    // waves holding the tail state
    const bool tw = w < TW;
    bool sh_zero = false;         // the reverse state is known to be exactly zero
    if (tail > 0) {
        auto ttile = [&](int i) { return reinterpret_cast<T *>(smem + L::WORK + i * L::TILE); };
        T *Tq = ttile(0), *Tk = ttile(1), *Tv = ttile(2), *Tg = ttile(3);
        {
            Stager<T, D> a, b2, c2, d2;
            a.load(qres, tt0 * D, D, tid);  // rows past the chunk read as zero
            b2.load(kres, tt0 * D, D, tid);
            c2.load(vres, tt0 * D, D, tid);
            d2.load(gres, tt0 * D, D, tid);
            __syncthreads();  // the block phase is done with the work area and the state copies
#pragma unroll
            for (int pi = 0; pi < NPT; ++pi)
#pragma unroll
                for (int cc = 0; cc < NHT; ++cc)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Sf[(ptile(pi) + 4 * g + i) * L::LDSF + ctile(cc) + r] = Sacc[pi][cc][i];
            a.store(Tq, L::LDN, nullptr, 0, tid);
            b2.store(Tk, L::LDN, nullptr, 0, tid);
            c2.store(Tv, L::LDN, nullptr, 0, tid);
            d2.store(Tg, L::LDN, nullptr, 0, tid);
            __syncthreads();
        }
        // layout A: lane owns column cA = 16w + r, key features g*NP.. (as rows p)
        // layout B: lane owns row pB = 16w + r, value features g*NP.. (as columns c)
        const int wl = w;
        float SA[NH][NP], SB[NH][NP], zA[NP], zB[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int s = 0; s < NP; ++s) {
                SA[h][s] = Sf[(g * NP + s) * L::LDSF + 64 * h + 16 * wl + r];
                SB[h][s] = Sf[(64 * h + 16 * wl + r) * L::LDSF + g * NP + s];
            }
#pragma unroll
        for (int s = 0; s < NP; ++s) zA[s] = zs[g * NP + s];
#pragma unroll
        for (int h = 0; h < NH; ++h) zB[h] = zs[64 * h + 16 * wl + r];

        // ---- pass 1 tail: forward order
        for (int t = 0; t < tail; ++t) {
            const T *qt = Tq + t * L::LDN, *kt = Tk + t * L::LDN, *vt = Tv + t * L::LDN, *gt = Tg + t * L::LDN;
            float inv = 0.f;
            if (tw) {
                float n[NH], d = 0.f, vA[NH];
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    n[h] = 0.f;
                    vA[h] = tof(vt[64 * h + 16 * wl + r]);
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
                inv = 1.f / d;
                float pd = 0.f;
#pragma unroll
                for (int h = 0; h < NH; ++h) pd += tof(gt[64 * h + 16 * wl + r]) * (wsum_g(n[h]) * inv);
                pd += __shfl_xor(pd, 1);
                pd += __shfl_xor(pd, 2);
                pd += __shfl_xor(pd, 4);
                pd += __shfl_xor(pd, 8);
                if (lane == 0) part[(t & 1) * NWAVE + w] = pd;
                if (tid == 0) den_all[tt0 + t] = d;
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    const float kp = tof(kt[64 * h + 16 * wl + r]);
                    zB[h] += kp;
#pragma unroll
                    for (int s = 0; s < NP; ++s) SB[h][s] += kp * tof(vt[g * NP + s]);
                }
            }
            __syncthreads();
            if (tw) {
                float rd = 0.f;
#pragma unroll
                for (int ww = 0; ww < TW; ++ww) rd += part[(t & 1) * NWAVE + ww];
                const float ddn = -rd * inv;
                if (tid == 0) dden_all[tt0 + t] = ddn;
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    float a = 0.f;
#pragma unroll
                    for (int s = 0; s < NP; ++s) a += SB[h][s] * tof(gt[g * NP + s]);
                    a = wsum_g(a) * inv + ddn * zB[h];
                    if (g == 0) dqg[(size_t)(tt0 + t) * D + 64 * h + 16 * wl + r] = fromf<T>(a);
                }
            }
        }

        // ---- pass 2 tail: reverse order, from the upstream carry gradient
        const GRes dSr = dS_out ? GRes(dS_out + (size_t)grp * D * D, D * D * 4) : none;
        const GRes dzr = dz_out ? GRes(dz_out + (size_t)grp * D, D * 4) : none;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
#pragma unroll
            for (int s = 0; s < NP; ++s) {
                SA[h][s] = gload<float>(dSr, ((g * NP + s) * D + 64 * h + 16 * wl + r) * 4);
                SB[h][s] = gload<float>(dSr, ((64 * h + 16 * wl + r) * D + g * NP + s) * 4);
            }
            zB[h] = gload<float>(dzr, (64 * h + 16 * wl + r) * 4);
        }
        __syncthreads();  // den_all / dden_all of the tail are visible
        if (tw) {
            for (int t = tail - 1; t >= 0; --t) {
                const T *qt = Tq + t * L::LDN, *kt = Tk + t * L::LDN, *vt = Tv + t * L::LDN, *gt = Tg + t * L::LDN;
                const float inv = 1.f / den_all[tt0 + t], ddn = dden_all[tt0 + t];
                float dnA[NH], a[NH];
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    dnA[h] = tof(gt[64 * h + 16 * wl + r]) * inv;
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
                    if (g == 0) dvg[(size_t)(tt0 + t) * D + 64 * h + 16 * wl + r] = fromf<T>(x);
                }
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    const float qp = tof(qt[64 * h + 16 * wl + r]);
                    zB[h] += ddn * qp;
                    float x = 0.f;
#pragma unroll
                    for (int s = 0; s < NP; ++s) {
                        SB[h][s] += qp * (tof(gt[g * NP + s]) * inv);
                        x += SB[h][s] * tof(vt[g * NP + s]);
                    }
                    x = wsum_g(x) + zB[h];
                    if (g == 0) dkg[(size_t)(tt0 + t) * D + 64 * h + 16 * wl + r] = fromf<T>(x);
                }
            }
        }
        if (nb == 0) {
            if (tw) {
                float *dSg = dS_in + (size_t)grp * D * D;
#pragma unroll
                for (int h = 0; h < NH; ++h)
#pragma unroll
                    for (int s = 0; s < NP; ++s) dSg[(size_t)(g * NP + s) * D + 64 * h + 16 * wl + r] = SA[h][s];
                if (g == 0) {
#pragma unroll
                    for (int h = 0; h < NH; ++h) dz_in[(size_t)grp * D + 64 * h + 16 * wl + r] = zB[h];
                }
            }
            return;
        }
        load_block(nxt, nb - 1, true);  // pass 2's first block
        __syncthreads();  // every wave is done with the tail tiles and pass 1's z
        if (tw) {
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int s = 0; s < NP; ++s) Sf[(g * NP + s) * L::LDSF + 64 * h + 16 * wl + r] = SA[h][s];
            if (g == 0) {
#pragma unroll
                for (int h = 0; h < NH; ++h) zs[64 * h + 16 * wl + r] = zB[h];
            }
        }
        __syncthreads();
#pragma unroll
        for (int pi = 0; pi < NPT; ++pi)
#pragma unroll
            for (int cc = 0; cc < NHT; ++cc)
#pragma unroll
                for (int i = 0; i < 4; ++i) Sacc[pi][cc][i] = Sf[(ptile(pi) + 4 * g + i) * L::LDSF + ctile(cc) + r];
        __syncthreads();  // the fp32 area aliases the copies written next
    } else {
        // no tail: the reverse state starts at the upstream carry gradient
        sh_zero = dS_out == nullptr;
        load_state(dS_out ? GRes(dS_out + (size_t)grp * D * D, D * D * 4) : none);
        const float dzo = gload<float>(dz_out ? GRes(dz_out + (size_t)grp * D, D * 4) : none, tid * 4);
        __syncthreads();  // pass 1 is done reading the state copies, the work area and z
        if (tid < D) zs[tid] = dzo;
    }
    write_copies();

    // =========================== pass 2: reverse sweep over blocks ===========================
    for (int b = nb - 1; b >= 0; --b) {
        const int t0 = b * BK, buf = TWOBUF ? (b & 1) : 0;
        const T *Qn = tile2(buf, 0), *Nh = tile2(buf, 1), *Nl = tile2(buf, 2);
        if (!TWOBUF && b < nb - 1) __syncthreads();  // one buffer: the previous update is done with it
        stage2(nxt, buf, b);
        Frag<T> fo[NKC];  // this wave's K rows (half 0) or V rows (half 1)
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) fo[kc] = nxt.f[kc];
        load_block(nxt, b > 0 ? b - 1 : past, true);
        __syncthreads();  // block staged; previous reverse-state update visible
        // dden_t per slot of the two 32-token chunks (slot s of chunk h: t = 32h + kslot)
        floatx8 dsl[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int s = 0; s < 8; ++s) dsl[h][s] = dden_all[t0 + 32 * h + kslot(lane, s)];

        const int jrow = t0 + 16 * tq + r;
        if (hh == 0) {
            // P[t][j] as acc(t, j) (lane: key j = 16tq + r, queries 16tt + 4g + i), then
            // dV^T[c][j] = dN^T P (intra) + Sh^T K^T (inter)
            floatx4 ap[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) ap[tt] = zero4();
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                Frag<T> qn[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) qn[tt] = ldfrag<T>(Qn + 16 * tt * L::LDN + 32 * kc, L::LDN, lane);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) mma(ap[tt], qn[tt], fo[kc]);
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool keep = tt > tq || (tt == tq && r <= 4 * g + i);  // key j <= query t
                    ap[tt][i] = keep ? ap[tt][i] : 0.f;
                }
            const SFrag<T> pa0 = split8<T>(acc8(ap[0], ap[1])), pa1 = split8<T>(acc8(ap[2], ap[3]));
            floatx4 av[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                av[ct] = zero4();
                mma_ss<T>(av[ct], ldsplit_tr<T>(Nh + 16 * ct, Nl + 16 * ct, L::LDN, lane), pa0);
                mma_ss<T>(av[ct], ldsplit_tr<T>(Nh + 32 * L::LDN + 16 * ct, Nl + 32 * L::LDN + 16 * ct, L::LDN, lane), pa1);
                if (!sh_zero) {
#pragma unroll
                    for (int kc = 0; kc < NKC; ++kc) {
                        const int off = 16 * ct * L::LDST + 32 * kc;
                        mma_sx<T>(av[ct], ldsplit<T>(STh + off, STl + off, L::LDST, lane), fo[kc]);
                    }
                }
            }
            T *vrow = dvg + (size_t)jrow * D + 4 * g;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) *reinterpret_cast<Vec4<T> *>(vrow + 16 * ct) = to_vec4<T>(av[ct]);
        } else {
            // dP[t][j] = dN V^T + dden as acc(t, j), then dK^T[p][j] = Q^T dP (intra) + Sh V^T + zh
            floatx4 ad[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) ad[tt] = zero4();
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                SFrag<T> dn[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int off = 16 * tt * L::LDN + 32 * kc;
                    dn[tt] = ldsplit<T>(Nh + off, Nl + off, L::LDN, lane);
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) mma_sx<T>(ad[tt], dn[tt], fo[kc]);
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool keep = tt > tq || (tt == tq && r <= 4 * g + i);
                    ad[tt][i] = keep ? ad[tt][i] + dden_all[t0 + 16 * tt + 4 * g + i] : 0.f;
                }
            const SFrag<T> pd0 = split8<T>(acc8(ad[0], ad[1])), pd1 = split8<T>(acc8(ad[2], ad[3]));
            floatx4 ak[NCT];
#pragma unroll
            for (int pt = 0; pt < NCT; ++pt) {
                ak[pt] = zero4();
                mma_xs<T>(ak[pt], ldfrag_tr<T>(Qn + 16 * pt, L::LDN, lane), pd0);
                mma_xs<T>(ak[pt], ldfrag_tr<T>(Qn + 32 * L::LDN + 16 * pt, L::LDN, lane), pd1);
                if (!sh_zero) {
#pragma unroll
                    for (int kc = 0; kc < NKC; ++kc) {
                        const int off = 32 * kc * L::LDST + 16 * pt;
                        mma_sx<T>(ak[pt], ldsplit_tr<T>(STh + off, STl + off, L::LDST, lane), fo[kc]);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) ak[pt][i] += zs[16 * pt + 4 * g + i];
                }
            }
            T *krow = dkg + (size_t)jrow * D + 4 * g;
#pragma unroll
            for (int pt = 0; pt < NCT; ++pt) *reinterpret_cast<Vec4<T> *>(krow + 16 * pt) = to_vec4<T>(ak[pt]);
        }
        __syncthreads();  // every wave is done reading the reverse-state copies and zh
        // Sh += Q^T dN, zh += Q^T dden (this wave: p-tiles tq + 4*pi, this half's c-tiles)
#pragma unroll
        for (int pi = 0; pi < NPT; ++pi) {
            const int p0 = ptile(pi);
            const Frag<T> qa = ldfrag_tr<T>(Qn + p0, L::LDN, lane);
            const Frag<T> qb = ldfrag_tr<T>(Qn + 32 * L::LDN + p0, L::LDN, lane);
#pragma unroll
            for (int cc = 0; cc < NHT; ++cc) {
                const int c0 = ctile(cc);
                mma_xs<T>(Sacc[pi][cc], qa, ldsplit_tr<T>(Nh + c0, Nl + c0, L::LDN, lane));
                mma_xs<T>(Sacc[pi][cc], qb, ldsplit_tr<T>(Nh + 32 * L::LDN + c0, Nl + 32 * L::LDN + c0, L::LDN, lane));
            }
            if (hh == 0) {
                floatx4 zacc = zero4();
                mma_xs<T>(zacc, qa, split8<T>(dsl[0]));
                mma_xs<T>(zacc, qb, split8<T>(dsl[1]));
                if (r == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) zs[p0 + 4 * g + i] += zacc[i];
                }
            }
        }
        if (b > 0) write_copies();
        sh_zero = false;
    }
    float *dSg = dS_in + (size_t)grp * D * D;
#pragma unroll
    for (int pi = 0; pi < NPT; ++pi)
#pragma unroll
        for (int cc = 0; cc < NHT; ++cc)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dSg[(size_t)(ptile(pi) + 4 * g + i) * D + ctile(cc) + r] = Sacc[pi][cc][i];
    __syncthreads();
    if (tid < D) dz_in[(size_t)grp * D + tid] = zs[tid];
}

template <typename T, int D>
hipError_t launch_bwd(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                      const void *dO, const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv,
                      float *dS_in, float *dz_in, int G, int C, hipStream_t stream,
                      const hipEvent_t ev[2]) {
    hipExtLaunchKernelGGL((la_bwd_kernel<T, D>), dim3((unsigned)G), dim3(NTHR), 0, stream, ev[0], ev[1], 0,
                          (const T *)q, (const T *)k, (const T *)v, S_in, z_in, (const T *)dO, dS_out, dz_out,
                          (T *)dq, (T *)dk, (T *)dv, dS_in, dz_in, C);
    return hipGetLastError();
}

template hipError_t launch_bwd<float, 64>(const void *, const void *, const void *, const float *, const float *,
                                          const void *, const float *, const float *, void *, void *, void *,
                                          float *, float *, int, int, hipStream_t, const hipEvent_t *);
template hipError_t launch_bwd<bf16, 64>(const void *, const void *, const void *, const float *, const float *,
                                         const void *, const float *, const float *, void *, void *, void *,
                                         float *, float *, int, int, hipStream_t, const hipEvent_t *);
template hipError_t launch_bwd<bf16, 128>(const void *, const void *, const void *, const float *, const float *,
                                          const void *, const float *, const float *, void *, void *, void *,
                                          float *, float *, int, int, hipStream_t, const hipEvent_t *);

}  // namespace lachunk
