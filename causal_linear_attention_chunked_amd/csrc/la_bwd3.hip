// Backward kernel for 128-token bf16 chunks at D = 64: the reverse scan of
// "Fractus-1B training optimization" (section 1: the gradient of a prefix sum is a
// suffix sum) over the blocked form of section 2, Opt 2, one workgroup per group.
//
// Loss L = sum_t <dO_t, o_t> + <dS_out, S_out> + dz_out . z_out.  Block b has the
// forward state S_b, z_b before it (S_0 = S_in, S_1 = S_0 + K_0^T V_0) and the reverse
// state Sh_b, zh_b after it (Sh_1 = dS_out, Sh_0 = Sh_1 + Q_1^T dN_1).  Per query t of
// block b, with A = Q K^T and G = dO V^T masked to j <= t and H_t = S_b dO_t:
//   den_t = sum_j A_tj + q_t . z_b          inv_t = 1 / den_t
//   rho_t = inv_t (sum_j A_tj G_tj + q_t . H_t)      (= dO_t . o_t)
//   dden_t = -rho_t inv_t,   dN_t = inv_t dO_t,   dP_tj = inv_t (G_tj - rho_t)
//   dq_t  = sum_j dP_tj k_j + inv_t H_t + dden_t z_b
//   dk_j  = sum_{t>=j} dP_tj q_t + Sh_b v_j + zh_b
//   dv_j  = sum_{t>=j} A_tj inv_t dO_t + Sh_b^T k_j
//   dS_in = Sh_0 + Q_0^T dN_0,   dz_in = zh_0 + Q_0^T dden_0   (zh likewise with dden)
// The row statistics den and rho come from fp32 accumulators (A, G exact products of
// the bf16 inputs), so the scores never enter a second product in pass 1.  fp32
// intermediates that are MFMA operands (S_b, dP, A inv, dN, Sh) are split hi + lo.
//
// Phases (8 waves, two per SIMD), separated by barriers:
//   0  stage Q, K, V, dO; split copies of S_0 and Sh_1; z_0, zh_1
//   1  S_1 (split copy, z_1); A and G tiles of the wave's query tile
//   2  H, den, rho; dP (split, kept in LDS for pass 2), dq stored; inv, rho, dden kept
//   3  reverse state Sh_0 = Sh_1 + Q_1^T dN_1 (split copy), zh_0; pass 2 of block 1 and
//      the intra-block part of pass 2 of block 0
//   4  the inter-block part of block 0 against Sh_0; dS_in = Sh_0 + Q_0^T dN_0 stored
// Waves: pass 1 on (block w/4, query tile, the second block's tiles reversed); state
// tiles (value tile w%4, key-feature tiles w/4, w/4 + 2); pass 2 on key tile w%4, dv
// for waves 0-3 and dk for waves 4-7, both blocks.
#include "la_tile.h"
#include "la_launch.h"
#include <hip/hip_ext.h>

namespace lachunk {

namespace {
struct Bwd3Lds {
    static constexpr int QT = 0;                 // Q[2], K[2], V[2], dO[2] tiles
    static constexpr int KT = QT + 2 * TBYTES;
    static constexpr int VT = KT + 2 * TBYTES;
    static constexpr int GT = VT + 2 * TBYTES;
    static constexpr int SS = GT + 2 * TBYTES;   // [b][hi, lo] split S_b; from phase 3: Sh_0 [hi, lo]
    static constexpr int SH1 = SS + 4 * TBYTES;  // Sh_1 [hi, lo]
    static constexpr int DP = SH1 + 2 * TBYTES;  // [b][hi, lo] split dP, stored [t][j]
    static constexpr int ZF = DP + 4 * TBYTES;   // [b][64] z_b fp32
    static constexpr int ZH = ZF + 2 * 64 * 4;   // [b][64] zh_b fp32
    static constexpr int INV = ZH + 2 * 64 * 4;  // [128] inv_t
    static constexpr int RHO = INV + 128 * 4;    // [128] rho_t
    static constexpr int DDR = RHO + 128 * 4;    // [hi, lo][128] dden_t bf16
    static constexpr int BYTES = DDR + 2 * 128 * 2;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};
}  // namespace

__global__ __launch_bounds__(NTHR, 1) void la_bwd_c128v3_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in, const bf16 *__restrict__ dO,
    const float *__restrict__ dS_out, const float *__restrict__ dz_out,
    bf16 *__restrict__ dq, bf16 *__restrict__ dk, bf16 *__restrict__ dv,
    float *__restrict__ dS_in, float *__restrict__ dz_in) {
    using L = Bwd3Lds;
    constexpr int D = 64, C = 128;
    constexpr uint32_t CHUNK = C * D * 2;
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    float *const zf = reinterpret_cast<float *>(smem + L::ZF);
    float *const zh = reinterpret_cast<float *>(smem + L::ZH);
    float *const invs = reinterpret_cast<float *>(smem + L::INV);
    float *const rhos = reinterpret_cast<float *>(smem + L::RHO);
    bf16 *const ddr = reinterpret_cast<bf16 *>(smem + L::DDR);
    auto tile = [&](int base, int b) -> char * { return smem + base + b * TBYTES; };

    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int blk = w >> 2;                        // pass 1: block and query tile
    const int tq = blk ? 3 - (w & 3) : (w & 3);
    const int ct = w & 3, pt0 = w >> 2;            // state tiles
    const int pt[2] = {pt0, pt0 + 2};
    const int jt = w & 3, is_dk = w >> 2;          // pass 2: key tile, output
    const int grp = blockIdx.x;
    const size_t tok0 = (size_t)grp * C;
    const bool has_up = dS_out != nullptr;
    const GRes qr(q + tok0 * D, CHUNK), kr(k + tok0 * D, CHUNK), vr(v + tok0 * D, CHUNK), gr(dO + tok0 * D, CHUNK);
    const float *const dummy = dS_in;  // a valid base for an empty range
    const GRes sres(S_in ? (const void *)(S_in + (size_t)grp * D * D) : dummy, S_in ? D * D * 4 : 0);
    const GRes zres(z_in ? (const void *)(z_in + (size_t)grp * D) : dummy, z_in ? D * 4 : 0);
    const GRes shres(has_up ? (const void *)(dS_out + (size_t)grp * D * D) : dummy, has_up ? D * D * 4 : 0);
    const GRes zhres(dz_out ? (const void *)(dz_out + (size_t)grp * D) : dummy, dz_out ? D * 4 : 0);
    const TileLanes TL(lane);
    const uint32_t tr_c = TL.tr_at(ct), tr_p[2] = {TL.tr_at(pt0), TL.tr_at(pt0 + 2)}, nat_c = TL.nat_at(ct);

    // ---- prologue: every load issued before anything waits
    bf16x8 st[8];  // Q0 Q1 K0 K1 V0 V1 dO0 dO1, 16 bytes per thread each
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        st[0 + b] = gload<bf16x8>(qr, b * TBYTES + tid * 16);
        st[2 + b] = gload<bf16x8>(kr, b * TBYTES + tid * 16);
        st[4 + b] = gload<bf16x8>(vr, b * TBYTES + tid * 16);
        st[6 + b] = gload<bf16x8>(gr, b * TBYTES + tid * 16);
    }
    // state accumulators C[c][p] (lane: p = 16 pt[i] + r, c = 16 ct + 4g + e): S and Sh
    floatx4 Sacc[2], Sh[2], zr[2], zhr[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t so = ((16 * pt[i] + r) * D + 16 * ct + 4 * g) * 4;
        Sacc[i] = gload<floatx4>(sres, so);
        Sh[i] = gload<floatx4>(shres, so);
        const float a = ct == 0 ? gload<float>(zres, (16 * pt[i] + r) * 4) : 0.f;
        const float b = ct == 0 ? gload<float>(zhres, (16 * pt[i] + r) * 4) : 0.f;
        zr[i] = floatx4{a, a, a, a};
        zhr[i] = floatx4{b, b, b, b};
    }
    issue_fence();

    // ---- phase 0
    {
        const uint32_t so = stage_off(tid);
        constexpr int bases[4] = {L::QT, L::KT, L::VT, L::GT};
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int b = 0; b < 2; ++b) *reinterpret_cast<bf16x8 *>(tile(bases[x], b) + so) = st[2 * x + b];
    }
    // split copy of a state held as C[c][p] accumulators, stored [p][c] (hi tile, lo tile)
    auto write_split = [&](char *hi, char *lo, const floatx4 (&acc)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            bf16x4 h, l;
            split4(acc[i], h, l);
            tstore_acc(hi, nat_c, pt[i], h);
            tstore_acc(lo, nat_c, pt[i], l);
        }
    };
    auto write_z = [&](float *dst, const floatx4 (&zz)[2]) {
        if (ct == 0 && g == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i) dst[16 * pt[i] + r] = zz[i][0];
        }
    };
    write_split(tile(L::SS, 0), tile(L::SS, 1), Sacc);
    write_z(zf, zr);
    if (has_up) write_split(tile(L::SH1, 0), tile(L::SH1, 1), Sh);
    write_z(zh + 64, zhr);
    __syncthreads();

    // ---- phase 1.  S_1 = S_0 + K_0^T V_0 as C[c][p] = sum_j V[j][c] K[j][p]; z_1 = z_0 + K_0^T 1
    const bf16x8 ones = ones_frag<bf16>();
    {
        bf16x8 vt[2], kt[2][2];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            vt[kc] = tfrag_tr(tile(L::VT, 0), tr_c, kc);
#pragma unroll
            for (int i = 0; i < 2; ++i) kt[kc][i] = tfrag_tr(tile(L::KT, 0), tr_p[i], kc);
        }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                mma(Sacc[i], vt[kc], kt[kc][i]);
                if (ct == 0) mma(zr[i], ones, kt[kc][i]);
            }
    }
    // pass-1 operands of this wave's queries (row t = r, k = feature)
    bf16x8 qf[2], df[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        qf[kc] = tfrag(tile(L::QT, blk), TL, tq, kc);
        df[kc] = tfrag(tile(L::GT, blk), TL, tq, kc);
    }
    // A^T, G^T tiles (lane: query t = r, key j = 16 jt + 4g + i), masked to j <= t
    floatx4 aT[4], gT[4];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
        aT[j4] = zero4();
        gT[j4] = zero4();
        if (j4 <= tq) {
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                mma(aT[j4], tfrag(tile(L::KT, blk), TL, j4, kc), qf[kc]);
                mma(gT[j4], tfrag(tile(L::VT, blk), TL, j4, kc), df[kc]);
            }
            if (j4 == tq) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool keep = 4 * g + e <= r;
                    aT[j4][e] = keep ? aT[j4][e] : 0.f;
                    gT[j4][e] = keep ? gT[j4][e] : 0.f;
                }
            }
        }
    }
    write_split(tile(L::SS, 2), tile(L::SS, 3), Sacc);
    write_z(zf + 64, zr);
    __syncthreads();

    // ---- phase 2.  H^T[p][t] = sum_c S_b[p][c] dO[t][c] (lane: t = r, p = 16 pt + 4g + i)
    floatx4 hT[4];
#pragma unroll
    for (int p4 = 0; p4 < 4; ++p4) {
        hT[p4] = zero4();
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const Split8 s{tfrag(tile(L::SS, 2 * blk), TL, p4, kc), tfrag(tile(L::SS, 2 * blk + 1), TL, p4, kc)};
            mma_s(hT[p4], s, df[kc]);
        }
    }
    // row statistics: den, and rho * den = sum_j A G + q . H
    floatx4 zv[4];
    float dpart = 0.f, rpart = 0.f;
#pragma unroll
    for (int p4 = 0; p4 < 4; ++p4) {
        zv[p4] = *reinterpret_cast<const floatx4 *>(zf + 64 * blk + 16 * p4 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float qv = (float)qf[p4 >> 1][4 * (p4 & 1) + e];
            dpart += qv * zv[p4][e];
            rpart += qv * hT[p4][e];
        }
    }
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
        if (j4 <= tq) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dpart += aT[j4][e];
                rpart += aT[j4][e] * gT[j4][e];
            }
        }
    }
    const float den = gsum(dpart);
    const float inv = __builtin_amdgcn_rcpf(den);
    const float rho = gsum(rpart) * inv;
    const float dden = -rho * inv;
    // dP^T[j][t] = inv (G - rho), masked; split, as the operand (row t, k = j) of dq and kept for pass 2
    Split8 dps[2];
#pragma unroll
    for (int jc = 0; jc < 2; ++jc) {
        if (2 * jc <= tq) {
            floatx4 d[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int j4 = 2 * jc + h;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool keep = j4 < tq || (j4 == tq && 4 * g + e <= r);
                    d[h][e] = keep ? (gT[j4][e] - rho) * inv : 0.f;
                }
            }
            dps[jc] = split_acc(d[0], d[1]);
            tstore_frag(tile(L::DP, 2 * blk), TL, tq, jc, dps[jc].hi);
            tstore_frag(tile(L::DP, 2 * blk + 1), TL, tq, jc, dps[jc].lo);
        }
    }
    // dq^T[p][t] = sum_j K^T[p][j] dP[t][j] + inv H^T[p][t] + dden z_b[p]
    {
        bf16 *dqrow = dq + (tok0 + 64 * blk + 16 * tq + r) * D + 4 * g;
#pragma unroll
        for (int p4 = 0; p4 < 4; ++p4) {
            floatx4 acc = hT[p4] * inv + dden * zv[p4];
#pragma unroll
            for (int jc = 0; jc < 2; ++jc)
                if (2 * jc <= tq) mma_s(acc, tfrag_tr(tile(L::KT, blk), TL.tr[p4], jc), dps[jc]);
            __builtin_nontemporal_store(pack4(acc), reinterpret_cast<bf16x4 *>(dqrow + 16 * p4));
        }
    }
    if (g == 0) {
        const int t = 64 * blk + 16 * tq + r;
        invs[t] = inv;
        rhos[t] = rho;
        bf16x2 h, l;
        split_pair(dden, 0.f, h, l);
        ddr[t] = h[0];
        ddr[128 + t] = l[0];
    }
    __syncthreads();

    // ---- phase 3.  Reverse state: Sh += Q_b^T dN_b as C[c][p] = sum_t dN[t][c] Q[t][p],
    // zh += Q_b^T dden_b; dN^T (operand rows c, k = t) from dO^T scaled by inv_t
    auto reverse = [&](int b) {
#pragma unroll
        for (int tc = 0; tc < 2; ++tc) {
            const floatx4 i0 = *reinterpret_cast<const floatx4 *>(invs + 64 * b + 32 * tc + 4 * g);
            const floatx4 i1 = *reinterpret_cast<const floatx4 *>(invs + 64 * b + 32 * tc + 16 + 4 * g);
            const bf16x8 x = tfrag_tr(tile(L::GT, b), tr_c, tc);
            const floatx4 a0{(float)x[0] * i0[0], (float)x[1] * i0[1], (float)x[2] * i0[2], (float)x[3] * i0[3]};
            const floatx4 a1{(float)x[4] * i1[0], (float)x[5] * i1[1], (float)x[6] * i1[2], (float)x[7] * i1[3]};
            const Split8 dn = split_acc(a0, a1);
            bf16x8 dd[2];
            if (ct == 0) {
                dd[0] = rowfrag(reinterpret_cast<const char *>(ddr + 64 * b), lane, tc);
                dd[1] = rowfrag(reinterpret_cast<const char *>(ddr + 128 + 64 * b), lane, tc);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const bf16x8 qt = tfrag_tr(tile(L::QT, b), tr_p[i], tc);
                mma_s(Sh[i], dn, qt);
                if (ct == 0) {
                    mma(zhr[i], dd[0], qt);
                    mma(zhr[i], dd[1], qt);
                }
            }
        }
    };
    reverse(1);
    write_split(tile(L::SS, 0), tile(L::SS, 1), Sh);  // Sh_0 (the S_0 copy is no longer read)
    write_z(zh, zhr);

    // pass 2 for key tile jt of block b: dv^T[c][j] (waves 0-3) or dk^T[p][j] (waves 4-7),
    // lane: key j = r, column 16 x + 4g + i
    auto pass2_intra = [&](int b, floatx4 (&acc)[4], bf16x8 (&kv)[2]) {
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[x] = zero4();
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) kv[kc] = tfrag(tile(is_dk ? L::VT : L::KT, b), TL, jt, kc);
#pragma unroll
        for (int tc = 0; tc < 2; ++tc) {
            if (2 * tc + 1 < jt) continue;  // every query of the slab precedes the key tile
            Split8 y;
            if (is_dk) {
                // dP rows j, k = t, from the pass-1 copy
                y = Split8{tfrag_tr(tile(L::DP, 2 * b), TL.tr_at(jt), tc), tfrag_tr(tile(L::DP, 2 * b + 1), TL.tr_at(jt), tc)};
            } else {
                // A[t][j] inv_t recomputed (lane: j = r, t = 32 tc + 16 h + 4g + i), masked to t >= j
                floatx4 at[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int t4 = 2 * tc + h;
                    at[h] = zero4();
                    if (t4 >= jt) {
#pragma unroll
                        for (int kc = 0; kc < 2; ++kc) mma(at[h], tfrag(tile(L::QT, b), TL, t4, kc), kv[kc]);
                        const floatx4 iv = *reinterpret_cast<const floatx4 *>(invs + 64 * b + 16 * t4 + 4 * g);
#pragma unroll
                        for (int e = 0; e < 4; ++e) at[h][e] = (t4 > jt || 4 * g + e >= r) ? at[h][e] * iv[e] : 0.f;
                    }
                }
                y = split_acc(at[0], at[1]);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x)
                mma_s(acc[x], tfrag_tr(tile(is_dk ? L::QT : L::GT, b), TL.tr[x], tc), y);
        }
    };
    // inter-block part against Sh (split, stored [p][c]) and zh
    auto pass2_inter = [&](int b, floatx4 (&acc)[4], const bf16x8 (&kv)[2], const char *shh, const char *shl) {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const Split8 s = is_dk ? Split8{tfrag(shh, TL, x, kc), tfrag(shl, TL, x, kc)}
                                       : Split8{tfrag_tr(shh, TL.tr[x], kc), tfrag_tr(shl, TL.tr[x], kc)};
                mma_s(acc[x], s, kv[kc]);
            }
    };
    auto pass2_store = [&](int b, floatx4 (&acc)[4]) {
        bf16 *row = (is_dk ? dk : dv) + (tok0 + 64 * b + 16 * jt + r) * D + 4 * g;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            floatx4 y = acc[x];
            if (is_dk) y += *reinterpret_cast<const floatx4 *>(zh + 64 * b + 16 * x + 4 * g);
            __builtin_nontemporal_store(pack4(y), reinterpret_cast<bf16x4 *>(row + 16 * x));
        }
    };
    floatx4 acc1[4], acc0[4];
    bf16x8 kv1[2], kv0[2];
    pass2_intra(1, acc1, kv1);
    if (has_up) pass2_inter(1, acc1, kv1, tile(L::SH1, 0), tile(L::SH1, 1));
    pass2_store(1, acc1);
    pass2_intra(0, acc0, kv0);
    __syncthreads();  // Sh_0, zh_0 visible

    // ---- phase 4
    pass2_inter(0, acc0, kv0, tile(L::SS, 0), tile(L::SS, 1));
    pass2_store(0, acc0);
    reverse(0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = 16 * pt[i] + r;
        __builtin_nontemporal_store(Sh[i], reinterpret_cast<floatx4 *>(dS_in + ((size_t)grp * D + p) * D + 16 * ct + 4 * g));
        if (ct == 0 && g == 0) __builtin_nontemporal_store(zhr[i][0], dz_in + (size_t)grp * D + p);
    }
}

hipError_t launch_bwd_c128(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                           const void *dO, const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv,
                           float *dS_in, float *dz_in, int G, hipStream_t stream, const hipEvent_t ev[2]) {
    hipExtLaunchKernelGGL(la_bwd_c128v3_kernel, dim3((unsigned)G), dim3(NTHR), 0, stream, ev[0], ev[1], 0,
                          (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, S_in, z_in, (const bf16 *)dO, dS_out,
                          dz_out, (bf16 *)dq, (bf16 *)dk, (bf16 *)dv, dS_in, dz_in);
    return hipGetLastError();
}

}  // namespace lachunk
