// Backward kernel for 128-token bf16 chunks at D = 64: the reverse scan of
// "Fractus-1B training optimization" (section 1: the gradient of a prefix sum
// is a suffix sum) over the chunked form of section 2, Opt 2, with both 64-token
// blocks of the chunk worked on side by side.
//
// Loss L = sum_t <dO_t, o_t> + <dS_out, S_out> + dz_out . z_out.  For block b with
// forward state S_b, z_b (before the block) and reverse state Sh_b, zh_b (every
// later block's contribution plus dS_out, dz_out):
//   den = A 1 + Q z_b,  num = A V + Q S_b,  inv = 1/den          (A = Q K^T masked, j <= t)
//   G   = dO V^T,  H = dO S_b^T                                  (exact bf16 dO: no split)
//   dden = -inv^2 rowdot(dO, num),  dN = inv dO
//   dP  = (inv G + dden 1^T) masked
//   dQ  = dP K + inv H + dden z_b^T
//   dV  = A^T dN + K Sh_b,   dK = dP^T Q + V Sh_b^T + 1 zh_b^T
//   Sh_0 = Sh_1 + Q_1^T dN_1,  dS_in = Sh_0 + Q_0^T dN_0 (and zh with dden)
// Only the state S_1 = S_in + K_0^T V_0 links the blocks going forward, and only
// Sh_0 going back, so both are formed first and the blocks' work runs in
// parallel: waves 0-3 on block 0, 4-7 on block 1, a wave per 16 queries (pass 1)
// or 16 keys (pass 2).  dN and dP are formed once, in pass 1, and handed to
// pass 2 through LDS as split (hi + lo) bf16 tiles, read back transposed.
#include "la_common.h"
#include "la_launch.h"
#include <hip/hip_ext.h>

namespace lachunk {

// LDS map (bytes).  Every tile is [64][LDN] bf16.  Pass 1 uses K, V, Q and the
// split S^T copies; pass 2 reuses the K/V space for dN and the S^T space for dP.
struct Bwd2Lds {
    static constexpr int LDN = 64 + 8;
    static constexpr int TILE = 64 * LDN * 2;
    static constexpr int KB = 0;                 // K[2]            | pass 2: dN hi[2]
    static constexpr int VB = KB + 2 * TILE;     // V[2]            | pass 2: dN lo[2]
    static constexpr int QB = VB + 2 * TILE;     // Q[2]            | kept
    static constexpr int STH = QB + 2 * TILE;    // S^T hi[2]       | pass 2: dP hi[2]
    static constexpr int STL = STH + 2 * TILE;   // S^T lo[2]       | pass 2: dP lo[2]
    static constexpr int SHH = STL + 2 * TILE;   // Sh^T hi[2]
    static constexpr int SHL = SHH + 2 * TILE;   // Sh^T lo[2]
    static constexpr int ZS = SHL + 2 * TILE;    // [2][64] z_b
    static constexpr int ZH = ZS + 2 * 64 * 4;   // [2][64] zh_b
    static constexpr int DDEN = ZH + 2 * 64 * 4; // [128] dden_t
    static constexpr int BYTES = DDEN + 128 * 4;
    static_assert(BYTES <= 160 * 1024, "backward LDS budget exceeded");
};

// Writes a fragment (16 rows x one k-chunk) to a "row, k contiguous" matrix: the inverse of ldfrag.
__device__ __forceinline__ void stfrag(bf16 *base, int ld, int lane, const bf16x8 &f) {
    bf16 *p = base + (lane & 15) * ld + 4 * (lane >> 4);
    *reinterpret_cast<bf16x4 *>(p) = __builtin_shufflevector(f, f, 0, 1, 2, 3);
    *reinterpret_cast<bf16x4 *>(p + 16) = __builtin_shufflevector(f, f, 4, 5, 6, 7);
}

// fp32 values x[kslot(lane, s)] of one k-chunk, the same for every row of the fragment
__device__ __forceinline__ floatx8 row8(const float *x, int lane) {
    const float *p = x + 4 * (lane >> 4);
    const floatx4 a = *reinterpret_cast<const floatx4 *>(p);
    const floatx4 b = *reinterpret_cast<const floatx4 *>(p + 16);
    return floatx8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__global__ __launch_bounds__(NTHR, 1) void la_bwd_c128_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in, const bf16 *__restrict__ dO,
    const float *__restrict__ dS_out, const float *__restrict__ dz_out,
    bf16 *__restrict__ dq, bf16 *__restrict__ dk, bf16 *__restrict__ dv,
    float *__restrict__ dS_in, float *__restrict__ dz_in) {
    using L = Bwd2Lds;
    constexpr int D = 64, C = 128, LDN = L::LDN, TE = 64 * LDN;  // TE: elements per tile
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    bf16 *Ks = reinterpret_cast<bf16 *>(smem + L::KB);
    bf16 *Vs = reinterpret_cast<bf16 *>(smem + L::VB);
    bf16 *Qs = reinterpret_cast<bf16 *>(smem + L::QB);
    bf16 *STh = reinterpret_cast<bf16 *>(smem + L::STH);
    bf16 *STl = reinterpret_cast<bf16 *>(smem + L::STL);
    bf16 *SHh = reinterpret_cast<bf16 *>(smem + L::SHH);
    bf16 *SHl = reinterpret_cast<bf16 *>(smem + L::SHL);
    bf16 *dNh = Ks, *dNl = Vs, *dPh = STh, *dPl = STl;  // pass 2 reuse
    float *zs = reinterpret_cast<float *>(smem + L::ZS);
    float *zh = reinterpret_cast<float *>(smem + L::ZH);
    float *ddn = reinterpret_cast<float *>(smem + L::DDEN);

    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // block of this wave and its 16-row tile (queries in pass 1, keys in pass 2); the
    // second block's tiles run in reverse so the two waves of a SIMD balance their causal work
    const int blk = w >> 2;
    const int tq = blk ? 3 - (w & 3) : (w & 3);
    // state tiles owned in both passes: value tile ct, key-feature tiles pt0 and pt0 + 2
    const int ct = w & 3, pt0 = w >> 2;
    const int grp = blockIdx.x;
    const size_t tok0 = (size_t)grp * C;
    constexpr uint32_t CHUNK = C * D * 2;
    const GRes qr(q + tok0 * D, CHUNK), kr(k + tok0 * D, CHUNK), vr(v + tok0 * D, CHUNK), gr(dO + tok0 * D, CHUNK);
    const float *const base_any = dS_in;  // a valid address for empty ranges
    const GRes sres(S_in ? (const void *)(S_in + (size_t)grp * D * D) : base_any, S_in ? D * D * 4 : 0);
    const GRes zres(z_in ? (const void *)(z_in + (size_t)grp * D) : base_any, z_in ? D * 4 : 0);
    const GRes shres(dS_out ? (const void *)(dS_out + (size_t)grp * D * D) : base_any, dS_out ? D * D * 4 : 0);
    const GRes zhres(dz_out ? (const void *)(dz_out + (size_t)grp * D) : base_any, dz_out ? D * 4 : 0);

    // ---- prologue: every input of the chunk is requested before anything waits
    Stager<bf16, 64> ks[2], vs[2], qs[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        ks[b].load(kr, b * 64 * D, D, tid);
        vs[b].load(vr, b * 64 * D, D, tid);
        qs[b].load(qr, b * 64 * D, D, tid);
    }
    bf16x8 dof[2];  // dO rows of this wave's query tile, k = value feature
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) dof[kc] = ldfrag_g<bf16>(gr, (blk * 64 + 16 * tq) * D + 32 * kc, D, lane);
    floatx4 Sacc[2], zr[2], Shacc[2], zhr[2];  // tiles (p-tile pt0 + 2i, c-tile ct); lane c = r, element p = 4g + e
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int p = 16 * (pt0 + 2 * i) + 4 * g + e;
            const uint32_t so = (p * D + 16 * ct + r) * 4;
            Sacc[i][e] = gload<float>(sres, so);
            Shacc[i][e] = gload<float>(shres, so);
            zr[i][e] = gload<float>(zres, p * 4);
            zhr[i][e] = gload<float>(zhres, p * 4);
        }
    __syncthreads();  // keeps every prologue load issued here, ahead of the first wait

    const bf16x8 ones = ones_frag<bf16>();
    // split S^T (or Sh^T) copy of the owned tiles, and z (or zh) by the waves of value tile 0
    auto write_copy = [&](bf16 *hi, bf16 *lo, float *zdst, const floatx4 (&acc)[2], const floatx4 (&zacc)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int off = (16 * ct + r) * LDN + 16 * (pt0 + 2 * i) + 4 * g;
            store_split4<bf16>(hi + off, lo + off, acc[i]);
            if (ct == 0 && r == 0) *reinterpret_cast<floatx4 *>(zdst + 16 * (pt0 + 2 * i) + 4 * g) = zacc[i];
        }
    };
    write_copy(STh, STl, zs, Sacc, zr);  // state before block 0
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        ks[b].store(Ks + b * TE, LDN, nullptr, 0, tid);
        vs[b].store(Vs + b * TE, LDN, nullptr, 0, tid);
        qs[b].store(Qs + b * TE, LDN, nullptr, 0, tid);
    }
    __syncthreads();  // K, V, Q and the block-0 state visible

    // ---- pass 1.  State before block 1: S_1 = S_0 + K_0^T V_0, z_1 = z_0 + K_0^T 1
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2) {
        const bf16x8 vt = ldfrag_tr<bf16>(Vs + 32 * kc2 * LDN + 16 * ct, LDN, lane);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const bf16x8 kt = ldfrag_tr<bf16>(Ks + 32 * kc2 * LDN + 16 * (pt0 + 2 * i), LDN, lane);
            mma(Sacc[i], kt, vt);
            if (ct == 0) mma(zr[i], kt, ones);
        }
    }
    write_copy(STh + TE, STl + TE, zs + 64, Sacc, zr);

    const bf16 *Kb = Ks + blk * TE, *Vb = Vs + blk * TE, *Qb = Qs + blk * TE;
    bf16x8 qc[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) qc[kc] = ldfrag<bf16>(Qb + 16 * tq * LDN + 32 * kc, LDN, lane);
    // scores P^T[j][t] (key tiles after the diagonal are zero), the intra-block numerator and
    // denominator, and G^T[j][t] = v_j . dO_t
    floatx4 sc[4], gt[4], nm[4], dn = zero4();
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        sc[jt] = zero4();
        gt[jt] = zero4();
        nm[jt] = zero4();
        if (jt <= tq) {
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                mma(sc[jt], ldfrag<bf16>(Kb + 16 * jt * LDN + 32 * kc, LDN, lane), qc[kc]);
                mma(gt[jt], ldfrag<bf16>(Vb + 16 * jt * LDN + 32 * kc, LDN, lane), dof[kc]);
            }
        }
        if (jt == tq) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sc[jt][e] = 4 * g + e <= r ? sc[jt][e] : 0.f;
        }
    }
    SFrag<bf16> pf[2];
    pf[0] = split8<bf16>(acc8(sc[0], sc[1]));
    mma_xs<bf16>(dn, ones, pf[0]);
#pragma unroll
    for (int c = 0; c < 4; ++c) mma_xs<bf16>(nm[c], ldfrag_tr<bf16>(Vb + 16 * c, LDN, lane), pf[0]);
    if (tq >= 2) {
        pf[1] = split8<bf16>(acc8(sc[2], sc[3]));
        mma_xs<bf16>(dn, ones, pf[1]);
#pragma unroll
        for (int c = 0; c < 4; ++c) mma_xs<bf16>(nm[c], ldfrag_tr<bf16>(Vb + 32 * LDN + 16 * c, LDN, lane), pf[1]);
    }
    __syncthreads();  // the block-1 state copy visible

    // inter-block terms against S_b: numerator, denominator and H^T[p][t] = (S_b dO_t)[p]
    const bf16 *STbh = STh + blk * TE, *STbl = STl + blk * TE;
    const float *zb = zs + 64 * blk;
    floatx4 ht[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) ht[pt] = zero4();
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        mma_sx<bf16>(dn, split8<bf16>(row8(zb + 32 * kc, lane)), qc[kc]);
#pragma unroll
        for (int c = 0; c < 4; ++c) mma(nm[c], ldfrag<bf16>(STbh + 16 * c * LDN + 32 * kc, LDN, lane), qc[kc]);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
            mma_sx<bf16>(ht[pt], ldsplit_tr<bf16>(STbh + 32 * kc * LDN + 16 * pt, STbl + 32 * kc * LDN + 16 * pt, LDN, lane),
                         dof[kc]);
    }
    const float inv = __builtin_amdgcn_rcpf(dn[0]);
    // rowdot(dO_t, num_t): slot s of chunk kc is value column 16 (2 kc + s/4) + 4 g + s%4
    float rd = 0.f;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int s = 0; s < 8; ++s) rd += tof(dof[kc][s]) * nm[2 * kc + (s >> 2)][s & 3];
    rd = wsum_g(rd);
    const float dden = -rd * inv * inv;
    if (g == 0) ddn[blk * 64 + 16 * tq + r] = dden;
    // dN = inv dO, split, for pass 2
    SFrag<bf16> dnf[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) dnf[kc] = split8<bf16>(tof8<bf16>(dof[kc]) * inv);
    // dP^T[j][t] = inv G^T + dden, masked; split
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool keep = jt < tq || (jt == tq && 4 * g + e <= r);
            gt[jt][e] = keep ? gt[jt][e] * inv + dden : 0.f;
        }
    }
    SFrag<bf16> dpf[2];
    dpf[0] = split8<bf16>(acc8(gt[0], gt[1]));
    dpf[1] = split8<bf16>(acc8(gt[2], gt[3]));
    // dQ^T[p][t] = K^T dP^T + inv H^T + dden z_b
    bf16 *dqrow = dq + (tok0 + blk * 64 + 16 * tq + r) * D + 4 * g;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
        const floatx4 z4 = *reinterpret_cast<const floatx4 *>(zb + 16 * pt + 4 * g);
        floatx4 acc = ht[pt] * inv + dden * z4;
        mma_xs<bf16>(acc, ldfrag_tr<bf16>(Kb + 16 * pt, LDN, lane), dpf[0]);
        if (tq >= 2) mma_xs<bf16>(acc, ldfrag_tr<bf16>(Kb + 32 * LDN + 16 * pt, LDN, lane), dpf[1]);
        *reinterpret_cast<bf16x4 *>(dqrow + 16 * pt) = to_vec4<bf16>(acc);
    }
    // pass-2 operands of this wave's key tile, taken before K and V are overwritten
    bf16x8 kf[2], vf[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        kf[kc] = ldfrag<bf16>(Kb + 16 * tq * LDN + 32 * kc, LDN, lane);
        vf[kc] = ldfrag<bf16>(Vb + 16 * tq * LDN + 32 * kc, LDN, lane);
    }
    __syncthreads();  // pass 1 is done with K, V and the S^T copies

    // ---- hand-over: dN and dP into LDS (natural [t][c] and [t][j]), the reverse state of block 1
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
        const int off = blk * TE + 16 * tq * LDN + 32 * kc;
        stfrag(dNh + off, LDN, lane, dnf[kc].hi);
        stfrag(dNl + off, LDN, lane, dnf[kc].lo);
        stfrag(dPh + off, LDN, lane, dpf[kc].hi);
        stfrag(dPl + off, LDN, lane, dpf[kc].lo);
    }
    write_copy(SHh + TE, SHl + TE, zh + 64, Shacc, zhr);  // Sh_1 = dS_out, zh_1 = dz_out
    __syncthreads();

    // ---- pass 2.  Reverse state before block 0: Sh_0 = Sh_1 + Q_1^T dN_1, zh_0 = zh_1 + Q_1^T dden_1
    auto reverse_update = [&](int b) {
#pragma unroll
        for (int tc = 0; tc < 2; ++tc) {
            const SFrag<bf16> dnt = ldsplit_tr<bf16>(dNh + b * TE + 32 * tc * LDN + 16 * ct,
                                                     dNl + b * TE + 32 * tc * LDN + 16 * ct, LDN, lane);
            SFrag<bf16> ddf;
            if (ct == 0) ddf = split8<bf16>(row8(ddn + 64 * b + 32 * tc, lane));
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const bf16x8 qt = ldfrag_tr<bf16>(Qs + b * TE + 32 * tc * LDN + 16 * (pt0 + 2 * i), LDN, lane);
                mma_xs<bf16>(Shacc[i], qt, dnt);
                if (ct == 0) mma_xs<bf16>(zhr[i], qt, ddf);
            }
        }
    };
    reverse_update(1);
    write_copy(SHh, SHl, zh, Shacc, zhr);

    // intra-block parts of dV^T[c][j] = dN^T A and dK^T[p][j] = Q^T dP for this wave's keys
    const int jt = tq;
    const bf16 *dNbh = dNh + blk * TE, *dNbl = dNl + blk * TE, *dPbh = dPh + blk * TE, *dPbl = dPl + blk * TE;
    floatx4 dva[4], dka[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        dva[c] = zero4();
        dka[c] = zero4();
    }
#pragma unroll
    for (int tc = 0; tc < 2; ++tc) {
        if (2 * tc + 1 < jt) continue;  // every query of this chunk precedes the keys
        // A^T[j][t] recomputed: rows j of this wave, queries of tiles 2tc, 2tc+1
        floatx4 at[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int tt = 2 * tc + h;
            at[h] = zero4();
            if (tt >= jt) {
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) mma(at[h], ldfrag<bf16>(Qb + 16 * tt * LDN + 32 * kc, LDN, lane), kf[kc]);
            }
            if (tt == jt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) at[h][e] = 4 * g + e >= r ? at[h][e] : 0.f;
            }
        }
        const SFrag<bf16> af = split8<bf16>(acc8(at[0], at[1]));
        const SFrag<bf16> dpt = ldsplit_tr<bf16>(dPbh + 32 * tc * LDN + 16 * jt, dPbl + 32 * tc * LDN + 16 * jt, LDN, lane);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            mma_ss<bf16>(dva[c], ldsplit_tr<bf16>(dNbh + 32 * tc * LDN + 16 * c, dNbl + 32 * tc * LDN + 16 * c, LDN, lane),
                         af);
            mma_xs<bf16>(dka[c], ldfrag_tr<bf16>(Qb + 32 * tc * LDN + 16 * c, LDN, lane), dpt);
        }
    }
    // inter-block parts against Sh_b: dV^T += Sh^T K^T, dK^T += Sh V^T + zh; then store
    auto inter_and_store = [&]() {
        const bf16 *SHbh = SHh + blk * TE, *SHbl = SHl + blk * TE;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                mma_sx<bf16>(dva[c], ldsplit<bf16>(SHbh + 16 * c * LDN + 32 * kc, SHbl + 16 * c * LDN + 32 * kc, LDN, lane),
                             kf[kc]);
                mma_sx<bf16>(dka[c], ldsplit_tr<bf16>(SHbh + 32 * kc * LDN + 16 * c, SHbl + 32 * kc * LDN + 16 * c, LDN, lane),
                             vf[kc]);
            }
        const size_t row = (tok0 + blk * 64 + 16 * jt + r) * D + 4 * g;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const floatx4 z4 = *reinterpret_cast<const floatx4 *>(zh + 64 * blk + 16 * c + 4 * g);
            *reinterpret_cast<bf16x4 *>(dv + row + 16 * c) = to_vec4<bf16>(dva[c]);
            *reinterpret_cast<bf16x4 *>(dk + row + 16 * c) = to_vec4<bf16>(dka[c] + z4);
        }
    };
    if (blk == 1) inter_and_store();  // Sh_1 was visible before this pass began
    __syncthreads();                   // Sh_0 visible
    if (blk == 0) inter_and_store();

    // dS_in = Sh_0 + Q_0^T dN_0, dz_in = zh_0 + Q_0^T dden_0
    reverse_update(0);
    float *Sg = dS_in + (size_t)grp * D * D + 16 * ct + r;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) Sg[(size_t)(16 * (pt0 + 2 * i) + 4 * g + e) * D] = Shacc[i][e];
    if (ct == 0 && r == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            *reinterpret_cast<floatx4 *>(dz_in + (size_t)grp * D + 16 * (pt0 + 2 * i) + 4 * g) = zhr[i];
    }
}

hipError_t launch_bwd_c128(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                           const void *dO, const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv,
                           float *dS_in, float *dz_in, int G, hipStream_t stream, const hipEvent_t ev[2]) {
    hipExtLaunchKernelGGL(la_bwd_c128_kernel, dim3((unsigned)G), dim3(NTHR), 0, stream, ev[0], ev[1], 0,
                          (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, S_in, z_in, (const bf16 *)dO, dS_out,
                          dz_out, (bf16 *)dq, (bf16 *)dk, (bf16 *)dv, dS_in, dz_in);
    return hipGetLastError();
}

}  // namespace lachunk
