// Sequence backward at D = 128 (bf16): the reverse scan of "Fractus-1B training
// optimization" (section 1: the gradient of a prefix sum is a suffix sum) over the
// blocked form of section 2, Opt 2, for a whole sequence of T tokens per group, one
// workgroup of 16 waves per group walking its 64-token blocks last to first.
//
// Per block b (the last one possibly ragged), with S_b, z_b the forward state before
// it and Sh_b, zh_b the reverse state after it (dS_out and dz_out plus every later
// token's contribution), A = Q K^T and G = dO V^T masked to j <= t, H_t = S_b dO_t:
//   den_t = sum_j A_tj + q_t . z_b          inv_t = 1 / den_t
//   rho_t = inv_t (sum_j A_tj G_tj + q_t . H_t)      (= dO_t . o_t)
//   dden_t = -rho_t inv_t,   dN_t = inv_t dO_t,   dP_tj = inv_t (G_tj - rho_t)
//   dq_t  = sum_j dP_tj k_j + inv_t H_t + dden_t z_b
//   dk_j  = sum_{t>=j} dP_tj q_t + Sh_b v_j + zh_b
//   dv_j  = sum_{t>=j} A_tj inv_t dO_t + Sh_b^T k_j
//   Sh_{b-1} = Sh_b + Q_b^T dN_b,   zh_{b-1} = zh_b + Q_b^T dden_b
// and dS_in, dz_in are the reverse state before the first block.
//
// The forward state is not stored by the forward pass: it is recovered from the
// carry after the last token, S_b = S_{b+1} - K_b^T V_b and z_b = z_{b+1} - K_b^T 1
// (exact products of the inputs, summed in fp32).  z is kept as an unevaluated sum
// with a compensation term (two-difference), starting from the final carry's remainder
// z_res: it grows with every token and the early normalisers are small next to the
// final one.  S starts from the carry and its remainder rounded once and is recovered
// in plain fp32 (no registers for a compensation term), which bounds the length.
//
// Registers hold the two D x D states (fp32, four 16 x 16 tiles per wave), LDS one
// split (hi + lo bf16) copy of a state at a time: S_b while the row statistics are
// formed, then Sh_b while the key-side gradients are.  Phases, separated by LDS-only
// barriers:
//   0  stage Q, K, V, dO of the block (loaded during the block before)
//   1  S_b (split copy), z_b; A, G of the wave's (query tile, key tile) pair
//   2  H for the wave's two key-feature tiles; partial row sums
//   3  den, rho, inv, dden; dP (split, stored [t][j]); Sh_b split copy, zh_b
//   4  dq; dv or dk of the wave's (key tile, column half); Sh_{b-1}, zh_{b-1}
// Rows past the end of the sequence read as zero, get inv = 0 and are not stored.
// FROM_IN (the one-chunk entry point, whose caller holds the carry before the chunk, not after
// it): the carry after the last token is first built from the carry before the first, S_in +
// sum_b K_b^T V_b over the blocks in order (z with a two-sum), the next block's keys and values
// loaded while one block's are added; the reverse walk then recovers the states from it as above.
// FM: q and k are raw inputs, mapped by elu(x) + 1 as they are staged; dq and dk are the
// gradients of the raw inputs, scaled at their stores by phi'(x) = min(1, phi) read back from the
// mapped tiles.  Mapped rows past the end of the sequence are zero, as raw ones are (phi(0) = 1
// would count the keys in the recovered z).
#include "la_tile.h"
#include "la_launch.h"
#include <hip/hip_ext.h>

namespace lachunk {

namespace {
constexpr int S128_THREADS = 1024;

struct Seq128Lds {
    static constexpr int QT = 0;                  // Q, K, V, dO of the block: two tiles each
    static constexpr int KT = QT + 2 * TBYTES;    //   (feature halves), rows = tokens
    static constexpr int VT = KT + 2 * TBYTES;
    static constexpr int GT = VT + 2 * TBYTES;
    static constexpr int SS = GT + 2 * TBYTES;    // state copy: hi tiles [pf][cf], then lo tiles
    static constexpr int DP = SS + 8 * TBYTES;    // dP hi, lo, stored [t][j]
    static constexpr int ZF = DP + 2 * TBYTES;    // [128] z_b fp32
    static constexpr int ZH = ZF + 128 * 4;       // [128] zh_b fp32
    static constexpr int INV = ZH + 128 * 4;      // [64] inv_t
    static constexpr int DDR = INV + 64 * 4;      // [hi, lo][64] dden_t bf16
    static constexpr int PS = DDR + 2 * 64 * 2;   // [16 waves][16 rows] (den, rho den) partials
    // the carried z (value and compensation) and zh, each entry read and written by its owner lane
    static constexpr int ZR = PS + 16 * 16 * 8, ZC = ZR + 128 * 4, ZHR = ZC + 128 * 4;
    static constexpr int BYTES = ZHR + 128 * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Key tile of the (A, G, dP) pair of the wave in query tile tq, slot s (its SIMD): every
// pair (tq, key) is covered once, and the pairs with work (key <= tq) are spread 2, 2, 3, 3
// over the four SIMDs.  Two bits per wave, wave w = 4 tq + s.
constexpr uint32_t key_table() {
    constexpr int t[16] = {1, 2, 3, 0, 2, 3, 0, 1, 0, 1, 2, 3, 0, 1, 2, 3};
    uint32_t x = 0;
    for (int i = 0; i < 16; ++i) x |= (uint32_t)t[i] << (2 * i);
    return x;
}
}  // namespace

template <bool FM, bool FROM_IN>
__device__ __forceinline__ void bwd_seq128_body(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_last, const float *__restrict__ z_last, const float *__restrict__ S_res,
    const float *__restrict__ z_res, const bf16 *__restrict__ dO,
    const float *__restrict__ dS_out, const float *__restrict__ dz_out,
    bf16 *__restrict__ dq, bf16 *__restrict__ dk, bf16 *__restrict__ dv,
    float *__restrict__ dS_in, float *__restrict__ dz_in, int T) {
    using L = Seq128Lds;
    constexpr int D = 128;
    constexpr uint32_t BLOCK = BK * D * 2;  // bytes of one block of one token tensor
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    float *const zf = reinterpret_cast<float *>(smem + L::ZF);
    float *const zh = reinterpret_cast<float *>(smem + L::ZH);
    float *const invs = reinterpret_cast<float *>(smem + L::INV);
    bf16 *const ddr = reinterpret_cast<bf16 *>(smem + L::DDR);
    floatx2 *const psum = reinterpret_cast<floatx2 *>(smem + L::PS);
    auto tq_ = [&](int base, int f) -> char * { return smem + base + f * TBYTES; };
    auto ssh = [&](int pf, int cf) -> char * { return smem + L::SS + (2 * pf + cf) * TBYTES; };
    auto ssl = [&](int pf, int cf) -> char * { return smem + L::SS + (4 + 2 * pf + cf) * TBYTES; };
    char *const dph = smem + L::DP, *const dpl = smem + L::DP + TBYTES;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // state role: value tile ct (feature half cf, tile cl in it), key-feature tiles pt0 + 2i
    // (i = 0..3: half i / 2, tile pt0 + 2 (i % 2) in it).  The waves with ct = 0 carry z and zh;
    // rotating ct by pt0 puts them on different SIMDs.
    const int pt0 = w >> 3, ct = (w + pt0) & 7, cf = ct >> 2, cl = ct & 3;
    // pass 1: query tile tq, slot s; key tile jt of the (A, G, dP) pair; key-feature tiles 2s, 2s + 1
    const int tq = w >> 2, s = w & 3;
    const int jt = (key_table() >> (2 * w)) & 3;
    // pass 2: dv (w < 8) or dk of key tile jt2 over the output's columns 64 oh..64 oh + 63; each
    // SIMD holds all four key tiles (long and short causal ranges)
    const int p2dk = w >> 3, oh = (w >> 2) & 1, jt2 = (w + (w >> 2)) & 3;

    const int grp = blockIdx.x;
    const size_t gtok0 = (size_t)grp * T;
    const uint32_t seq_bytes = (uint32_t)T * D * 2;
    const GRes qr(q + gtok0 * D, seq_bytes), kr(k + gtok0 * D, seq_bytes), vr(v + gtok0 * D, seq_bytes),
        gr(dO + gtok0 * D, seq_bytes);
    const float *const dummy = dS_in;  // a valid base for an empty range
    // S_last, z_last: the carry after the last token, or with FROM_IN the carry before the first (NULL
    // together: a zero carry)
    const GRes sres(S_last ? (const void *)(S_last + (size_t)grp * D * D) : dummy, S_last ? D * D * 4 : 0);
    const GRes zres(z_last ? (const void *)(z_last + (size_t)grp * D) : dummy, z_last ? D * 4 : 0);
    const GRes shres(dS_out ? (const void *)(dS_out + (size_t)grp * D * D) : dummy, dS_out ? D * D * 4 : 0);
    const GRes zhres(dz_out ? (const void *)(dz_out + (size_t)grp * D) : dummy, dz_out ? D * 4 : 0);
    const GRes srres(S_res ? (const void *)(S_res + (size_t)grp * D * D) : dummy, S_res ? D * D * 4 : 0);
    const GRes zrres(z_res ? (const void *)(z_res + (size_t)grp * D) : dummy, z_res ? D * 4 : 0);
    const int nblk = (T + BK - 1) / BK;

    // ---- prologue: the last block and both carries, every load issued before anything waits.
    // Thread tid stages 16 bytes of each tensor: token row tid / 16, feature half (tid / 8) % 2.
    bf16x8 st[4];
    auto load_stage = [&](int b) {
        const uint32_t o = (uint32_t)b * BLOCK + tid * 16;
        st[0] = gload<bf16x8>(qr, o);
        st[1] = gload<bf16x8>(kr, o);
        st[2] = gload<bf16x8>(vr, o);
        st[3] = gload<bf16x8>(gr, o);
    };
    load_stage(nblk - 1);
    // state accumulators C[c][p] (lane: p = 16 (pt0 + 2i) + r, c = 16 ct + 4g + e): S and Sh.
    // z and zh live in LDS (entry p owned by lane r = p % 16, g = 0 of a wave with ct = 0).
    float *const zrun = reinterpret_cast<float *>(smem + L::ZR);
    float *const zcmp = reinterpret_cast<float *>(smem + L::ZC);
    float *const zhrun = reinterpret_cast<float *>(smem + L::ZHR);
    floatx4 Sacc[4], Sh[4];
    {
        const int lane = tid & 63, r = lane & 15, g = lane >> 4;
        const bool zown = ct == 0 && g == 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = 16 * (pt0 + 2 * i) + r;
            const uint32_t so = (p * D + 16 * ct + 4 * g) * 4;
            // S starts from the final carry rounded once with its remainder (no compensation term
            // is carried for S here: registers); z from the carry and its remainder as they are
            Sacc[i] = gload<floatx4>(sres, so) + gload<floatx4>(srres, so);
            Sh[i] = gload<floatx4>(shres, so);
            const float z0 = gload<float>(zres, p * 4), zr0 = gload<float>(zrres, p * 4);
            const float zh0 = gload<float>(zhres, p * 4);
            if (zown) {
                zrun[p] = z0;
                zcmp[p] = zr0;
                zhrun[p] = zh0;
            }
        }
    }
    issue_fence();
    const bf16x8 ones = ones_frag<bf16>();

    if constexpr (FROM_IN) {
        // the carry after the last token: S += K_b^T V_b as C[c][p] = sum_j V[j][c] K[j][p] and z
        // += K_b^T 1 (two-sum), block by block in order; rows past the end read (and map) as zero
        const int row = tid >> 4, f = (tid >> 3) & 1;
        const uint32_t so = f * TBYTES + stage_off(row * 8 + (tid & 7));
        bf16x8 kx = gload<bf16x8>(kr, tid * 16), vx = gload<bf16x8>(vr, tid * 16);
        for (int b = 0; b < nblk; ++b) {
            const bool live = row < T - b * BK;
            *reinterpret_cast<bf16x8 *>(smem + L::KT + so) = FM ? (live ? elu1_8(kx) : bf16x8{}) : kx;
            *reinterpret_cast<bf16x8 *>(smem + L::VT + so) = vx;
            // the next block's, in flight during this one (past the range after the last: zeros)
            kx = gload<bf16x8>(kr, (uint32_t)(b + 1) * BLOCK + tid * 16);
            vx = gload<bf16x8>(vr, (uint32_t)(b + 1) * BLOCK + tid * 16);
            lds_barrier();
            const int lane = tid & 63, r = lane & 15, g = lane >> 4;
            const TileLanes TL(lane);
            const uint32_t tr_c = TL.tr_at(cl);
            bf16x8 vt[2];
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) vt[kc] = tfrag_tr(tq_(L::VT, cf), tr_c, kc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pf = i >> 1, pl = pt0 + 2 * (i & 1);
                bf16x8 kt[2];
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) kt[kc] = tfrag_tr(tq_(L::KT, pf), TL.tr_at(pl), kc);
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) mma(Sacc[i], vt[kc], kt[kc]);
                if (ct == 0) {
                    floatx4 Pz = zero4();
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc) mma(Pz, ones, kt[kc]);
                    if (g == 0) {
                        const int p = 16 * (pt0 + 2 * i) + r;
                        float zr = zrun[p], zc = zcmp[p];
                        two_sum(zr, zc, Pz[0]);
                        zrun[p] = zr;
                        zcmp[p] = zc;
                    }
                }
            }
            lds_barrier();  // the tiles are rewritten by the next block (or the first reverse step)
        }
    }

    for (int b = nblk - 1; b >= 0; --b) {
        // lane-dependent offsets derived afresh each block from an opaque copy of the thread index
        // (hoisted out of the loop they would all stay live across it)
        int tid_b = tid;
        asm volatile("" : "+v"(tid_b));
        const int lane = tid_b & 63, r = lane & 15, g = lane >> 4;
        const TileLanes TL(lane);
        const size_t tok0 = gtok0 + (size_t)b * BK;
        const int nvalid = T - b * BK;  // rows of this block inside the sequence (64 but for a ragged end)
        const bool has_up = b < nblk - 1 || dS_out != nullptr;

        // ---- phase 0
        {
            const int row = tid_b >> 4, f = (tid_b >> 3) & 1;
            const uint32_t so = f * TBYTES + stage_off(row * 8 + (tid_b & 7));
            const bool live = row < nvalid;
            *reinterpret_cast<bf16x8 *>(smem + L::QT + so) = FM ? (live ? elu1_8(st[0]) : bf16x8{}) : st[0];
            *reinterpret_cast<bf16x8 *>(smem + L::KT + so) = FM ? (live ? elu1_8(st[1]) : bf16x8{}) : st[1];
            *reinterpret_cast<bf16x8 *>(smem + L::VT + so) = st[2];
            *reinterpret_cast<bf16x8 *>(smem + L::GT + so) = st[3];
        }
        // the block before, in flight during this one (for b = 0 the offsets lie past the range:
        // zeros, no memory touched; a load on every path keeps the wait counts exact)
        load_stage(b - 1);
        lds_barrier();

        // ---- phase 1: S_b = S_{b+1} - K_b^T V_b as C[c][p] = sum_j V[j][c] K[j][p]; z likewise
        auto write_split = [&](char *hi, char *lo, const floatx4 &acc, int pl) {
            bf16x4 hh, ll;
            split4(acc, hh, ll);
            tstore_acc(hi, TL.nat_at(cl), pl, hh);
            tstore_acc(lo, TL.nat_at(cl), pl, ll);
        };
        {
            const uint32_t tr_c = TL.tr_at(cl);
            bf16x8 vt[2];
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) vt[kc] = tfrag_tr(tq_(L::VT, cf), tr_c, kc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pf = i >> 1, pl = pt0 + 2 * (i & 1);
                bf16x8 kt[2];
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) kt[kc] = tfrag_tr(tq_(L::KT, pf), TL.tr_at(pl), kc);
                floatx4 P = zero4();
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) mma(P, vt[kc], kt[kc]);
                Sacc[i] -= P;
                if (ct == 0) {
                    floatx4 Pz = zero4();
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc) mma(Pz, ones, kt[kc]);
                    if (g == 0) {
                        const int p = 16 * (pt0 + 2 * i) + r;
                        float zr = zrun[p], zc = zcmp[p];
                        two_diff(zr, zc, Pz[0]);
                        zrun[p] = zr;
                        zcmp[p] = zc;
                        zf[p] = zr + zc;
                    }
                }
                write_split(ssh(pf, cf), ssl(pf, cf), Sacc[i], pl);
            }
        }
        // A^T, G^T of key tile jt (lane: query t = 16 tq + r, key j = 16 jt + 4g + e), masked j <= t;
        // operands: rows of Q, dO (row t = r) and K, V (row j = r), k = feature / value column
        floatx4 aT = zero4(), gT = zero4();
        if (jt <= tq) {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                mma(aT, tfrag(tq_(L::KT, kc >> 1), TL, jt, kc & 1), tfrag(tq_(L::QT, kc >> 1), TL, tq, kc & 1));
                mma(gT, tfrag(tq_(L::VT, kc >> 1), TL, jt, kc & 1), tfrag(tq_(L::GT, kc >> 1), TL, tq, kc & 1));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool keep = jt < tq || 4 * g + e <= r;
                aT[e] = keep ? aT[e] : 0.f;
                gT[e] = keep ? gT[e] : 0.f;
            }
        }
        lds_barrier();

        // ---- phase 2: H^T[p][t] = sum_c S_b[p][c] dO[t][c] for key-feature tiles 2s + pp
        // (lane: t = r, p = 16 (2s + pp) + 4g + e; half s / 2, tile 2 (s % 2) + pp in it)
        floatx4 hT[2], zv[2];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) hT[pp] = zero4();
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            const bf16x8 dfr = tfrag(tq_(L::GT, kc >> 1), TL, tq, kc & 1);
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const int pf = s >> 1, pl = 2 * (s & 1) + pp;
                mma(hT[pp], tfrag(ssh(pf, kc >> 1), TL, pl, kc & 1), dfr);
                mma(hT[pp], tfrag(ssl(pf, kc >> 1), TL, pl, kc & 1), dfr);
            }
        }
        {
            // q_t[p] for p = 32 s + 16 pp + 4g + e: k-chunk s of the query fragments, slot 4 pp + e
            const bf16x8 qh = tfrag_at(tq_(L::QT, s >> 1), TL, tq, s & 1);
            float dpart = 0.f, rpart = 0.f;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                zv[pp] = *reinterpret_cast<const floatx4 *>(zf + 16 * (2 * s + pp) + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float qv = (float)qh[4 * pp + e];
                    dpart += qv * zv[pp][e];
                    rpart += qv * hT[pp][e];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dpart += aT[e];
                rpart += aT[e] * gT[e];
            }
            const float dsum = gsum(dpart), rsum = gsum(rpart);
            if (g == 0) psum[w * 16 + r] = floatx2{dsum, rsum};
        }
        lds_barrier();

        // ---- phase 3: row statistics from the four slots; dP of the wave's pair; Sh_b copy
        const bool valid = 16 * tq + r < nvalid;
        float inv, dden;
        {
            float den = 0.f, rr = 0.f;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const floatx2 pv = psum[(4 * tq + x) * 16 + r];
                den += pv[0];
                rr += pv[1];
            }
            inv = valid ? __builtin_amdgcn_rcpf(den) : 0.f;
            const float rho = rr * inv;
            dden = -rho * inv;
            floatx4 d;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool keep = jt < tq || (jt == tq && 4 * g + e <= r);
                d[e] = keep ? (gT[e] - rho) * inv : 0.f;
            }
            bf16x4 hh, ll;
            split4(d, hh, ll);
            tstore_acc(dph, TL.nat_at(jt), tq, hh);
            tstore_acc(dpl, TL.nat_at(jt), tq, ll);
            if (s == 0 && g == 0) {
                const int t = 16 * tq + r;
                invs[t] = inv;
                bf16x2 dh, dl;
                split_pair(dden, 0.f, dh, dl);
                ddr[t] = dh[0];
                ddr[64 + t] = dl[0];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pf = i >> 1, pl = pt0 + 2 * (i & 1);
            if (has_up) write_split(ssh(pf, cf), ssl(pf, cf), Sh[i], pl);
            if (ct == 0 && g == 0) zh[16 * (pt0 + 2 * i) + r] = zhrun[16 * (pt0 + 2 * i) + r];
        }
        lds_barrier();

        // ---- phase 4: dq^T[p][t] = sum_j K^T[p][j] dP[t][j] + inv H^T[p][t] + dden z_b[p]
        {
            bf16 *dqrow = dq + (tok0 + 16 * tq + r) * D + 4 * g;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const int pf = s >> 1, pl = 2 * (s & 1) + pp;
                floatx4 acc = hT[pp] * inv + dden * zv[pp];
#pragma unroll
                for (int jc = 0; jc < 2; ++jc) {
                    if (jc == 1 && tq < 2) continue;  // keys 32..63 follow every query of tiles 0, 1
                    const bf16x8 kx = tfrag_tr(tq_(L::KT, pf), TL.tr_at(pl), jc);
                    mma(acc, kx, tfrag(dph, TL, tq, jc));
                    mma(acc, kx, tfrag(dpl, TL, tq, jc));
                }
                // fused feature map: the raw query's gradient is dq phi'(x), phi' = min(1, phi)
                if constexpr (FM) acc *= elu1_grad4(lds_b64(tq_(L::QT, pf) + tq * 16 * TROW + TL.nat_at(pl)));
                if (valid) *reinterpret_cast<bf16x4 *>(dqrow + 16 * (2 * s + pp)) = pack4(acc);
            }
        }
        // pass 2: accumulators dv^T[c][j] or dk^T[p][j] (lane: key j = 16 jt2 + r, column
        // 64 oh + 16 x + 4g + e)
        {
            floatx4 acc[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) acc[x] = zero4();
            // rows j of K (dv: A recomputed, inter term over p) or of V (dk: inter term over c)
            auto kv = [&](int kc) { return tfrag(tq_(p2dk ? L::VT : L::KT, kc >> 1), TL, jt2, kc & 1); };
            const uint32_t tr_j = TL.tr_at(jt2);
#pragma unroll
            for (int tc = 0; tc < 2; ++tc) {
                if (2 * tc + 1 < jt2) continue;  // every query of the slab precedes the key tile
                Split8 y;
                if (p2dk) {
                    // dP rows j, k = t, from the phase-3 copy
                    y = Split8{tfrag_tr(dph, tr_j, tc), tfrag_tr(dpl, tr_j, tc)};
                } else {
                    // A[t][j] inv_t recomputed (lane: j = r, t = 32 tc + 16 hh + 4g + e), masked to t >= j
                    floatx4 at[2] = {zero4(), zero4()};
#pragma unroll
                    for (int kc = 0; kc < 4; ++kc) {
                        const bf16x8 kj = kv(kc);
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) mma(at[hh], tfrag(tq_(L::QT, kc >> 1), TL, 2 * tc + hh, kc & 1), kj);
                    }
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int t4 = 2 * tc + hh;
                        const floatx4 iv = *reinterpret_cast<const floatx4 *>(invs + 16 * t4 + 4 * g);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            at[hh][e] = (t4 > jt2 || (t4 == jt2 && 4 * g + e >= r)) ? at[hh][e] * iv[e] : 0.f;
                    }
                    y = split_acc(at[0], at[1]);
                }
                // dO^T rows c (dv) or Q^T rows p (dk) of this output half, k = t
#pragma unroll
                for (int x = 0; x < 4; ++x) mma_s(acc[x], tfrag_tr(tq_(p2dk ? L::QT : L::GT, oh), TL.tr[x], tc), y);
            }
            if (has_up) {
                // dv^T[c][j] += sum_p Sh[p][c] K[j][p]  (Sh^T rows c: transposed reads of the copy)
                // dk^T[p][j] += sum_c Sh[p][c] V[j][c]  (Sh rows p: natural reads)
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) {
                    const int kf = kc >> 1, k2 = kc & 1;
                    const bf16x8 kj = kv(kc);
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const bf16x8 a_hi = p2dk ? tfrag(ssh(oh, kf), TL, x, k2) : tfrag_tr(ssh(kf, oh), TL.tr[x], k2);
                        const bf16x8 a_lo = p2dk ? tfrag(ssl(oh, kf), TL, x, k2) : tfrag_tr(ssl(kf, oh), TL.tr[x], k2);
                        mma(acc[x], a_hi, kj);
                        mma(acc[x], a_lo, kj);
                    }
                }
            }
            if (16 * jt2 + r < nvalid) {
                bf16 *row = (p2dk ? dk : dv) + (tok0 + 16 * jt2 + r) * D + 64 * oh + 4 * g;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    floatx4 y = acc[x];
                    if (p2dk) {
                        y += *reinterpret_cast<const floatx4 *>(zh + 64 * oh + 16 * x + 4 * g);
                        if constexpr (FM) y *= elu1_grad4(lds_b64(tq_(L::KT, oh) + jt2 * 16 * TROW + TL.nat[x]));
                    }
                    *reinterpret_cast<bf16x4 *>(row + 16 * x) = pack4(y);
                }
            }
        }
        // reverse state: Sh += Q_b^T dN_b as C[c][p] = sum_t dN[t][c] Q[t][p], zh += Q_b^T dden_b;
        // dN^T (operand rows c, k = t) is dO^T scaled by inv_t
        {
            const uint32_t tr_c = TL.tr_at(cl);
#pragma unroll
            for (int tc = 0; tc < 2; ++tc) {
                const bf16x8 x = tfrag_tr(tq_(L::GT, cf), tr_c, tc);
                const floatx4 i0 = *reinterpret_cast<const floatx4 *>(invs + 32 * tc + 4 * g);
                const floatx4 i1 = *reinterpret_cast<const floatx4 *>(invs + 32 * tc + 16 + 4 * g);
                const floatx4 a0{(float)x[0] * i0[0], (float)x[1] * i0[1], (float)x[2] * i0[2], (float)x[3] * i0[3]};
                const floatx4 a1{(float)x[4] * i1[0], (float)x[5] * i1[1], (float)x[6] * i1[2], (float)x[7] * i1[3]};
                const Split8 dn = split_acc(a0, a1);
                bf16x8 drow[2];
                if (ct == 0) {
                    // the dden row (hi, lo) as an operand whose 16 rows are all that row
#pragma unroll
                    for (int hl = 0; hl < 2; ++hl) {
                        const bf16 *p = ddr + 64 * hl + 32 * tc + 4 * g;
                        drow[hl] = __builtin_shufflevector(lds_b64(reinterpret_cast<const char *>(p)),
                                                           lds_b64(reinterpret_cast<const char *>(p + 16)), 0, 1, 2,
                                                           3, 4, 5, 6, 7);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pf = i >> 1, pl = pt0 + 2 * (i & 1);
                    const bf16x8 qt = tfrag_tr(tq_(L::QT, pf), TL.tr_at(pl), tc);
                    mma_s(Sh[i], dn, qt);
                    if (ct == 0) {
                        floatx4 pz = zero4();
                        mma(pz, drow[0], qt);
                        mma(pz, drow[1], qt);
                        if (g == 0) zhrun[16 * (pt0 + 2 * i) + r] += pz[0];
                    }
                }
            }
        }
        // the tiles, the state copy and the small arrays are rewritten by the next block
        lds_barrier();
    }
    {
        const int lane = tid & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = 16 * (pt0 + 2 * i) + r;
            *reinterpret_cast<floatx4 *>(dS_in + ((size_t)grp * D + p) * D + 16 * ct + 4 * g) = Sh[i];
            if (ct == 0 && g == 0) dz_in[(size_t)grp * D + p] = zhrun[p];
        }
    }
}

__global__ __launch_bounds__(S128_THREADS, 1) void la_seq_bwd_d128_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_last, const float *__restrict__ z_last, const float *__restrict__ S_res,
    const float *__restrict__ z_res, const bf16 *__restrict__ dO,
    const float *__restrict__ dS_out, const float *__restrict__ dz_out,
    bf16 *__restrict__ dq, bf16 *__restrict__ dk, bf16 *__restrict__ dv,
    float *__restrict__ dS_in, float *__restrict__ dz_in, int T) {
    bwd_seq128_body<false, false>(q, k, v, S_last, z_last, S_res, z_res, dO, dS_out, dz_out, dq, dk, dv, dS_in, dz_in,
                                  T);
}

// the same with the feature map fused: dq and dk are the gradients of the raw inputs
__global__ __launch_bounds__(S128_THREADS, 1) void la_seq_bwd_d128_elu1_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_last, const float *__restrict__ z_last, const float *__restrict__ S_res,
    const float *__restrict__ z_res, const bf16 *__restrict__ dO,
    const float *__restrict__ dS_out, const float *__restrict__ dz_out,
    bf16 *__restrict__ dq, bf16 *__restrict__ dk, bf16 *__restrict__ dv,
    float *__restrict__ dS_in, float *__restrict__ dz_in, int T) {
    bwd_seq128_body<true, false>(q, k, v, S_last, z_last, S_res, z_res, dO, dS_out, dz_out, dq, dk, dv, dS_in, dz_in,
                                 T);
}

// One chunk of C tokens from the carry before it (the chunk entry point), with and without the map.
__global__ __launch_bounds__(S128_THREADS, 1) void la_bwd_d128_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in, const bf16 *__restrict__ dO,
    const float *__restrict__ dS_out, const float *__restrict__ dz_out,
    bf16 *__restrict__ dq, bf16 *__restrict__ dk, bf16 *__restrict__ dv,
    float *__restrict__ dS_in, float *__restrict__ dz_in, int C) {
    bwd_seq128_body<false, true>(q, k, v, S_in, z_in, nullptr, nullptr, dO, dS_out, dz_out, dq, dk, dv, dS_in, dz_in,
                                 C);
}

__global__ __launch_bounds__(S128_THREADS, 1) void la_bwd_d128_elu1_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in, const bf16 *__restrict__ dO,
    const float *__restrict__ dS_out, const float *__restrict__ dz_out,
    bf16 *__restrict__ dq, bf16 *__restrict__ dk, bf16 *__restrict__ dv,
    float *__restrict__ dS_in, float *__restrict__ dz_in, int C) {
    bwd_seq128_body<true, true>(q, k, v, S_in, z_in, nullptr, nullptr, dO, dS_out, dz_out, dq, dk, dv, dS_in, dz_in,
                                C);
}

hipError_t launch_bwd_d128(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                           const void *dO, const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv,
                           float *dS_in, float *dz_in, int G, int C, bool elu1, hipStream_t stream,
                           const hipEvent_t ev[2]) {
    hipExtLaunchKernelGGL(elu1 ? la_bwd_d128_elu1_kernel : la_bwd_d128_kernel, dim3((unsigned)G),
                          dim3(S128_THREADS), 0, stream, ev[0], ev[1], 0, (const bf16 *)q, (const bf16 *)k,
                          (const bf16 *)v, S_in, z_in, (const bf16 *)dO, dS_out, dz_out, (bf16 *)dq, (bf16 *)dk,
                          (bf16 *)dv, dS_in, dz_in, C);
    return hipGetLastError();
}

hipError_t launch_seq_bwd_d128(const void *q, const void *k, const void *v, const float *S_last,
                               const float *z_last, const float *S_res, const float *z_res, const void *dO,
                               const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv, float *dS_in,
                               float *dz_in, int G, int T, bool elu1, hipStream_t stream, const hipEvent_t ev[2]) {
    hipExtLaunchKernelGGL(elu1 ? la_seq_bwd_d128_elu1_kernel : la_seq_bwd_d128_kernel, dim3((unsigned)G),
                          dim3(S128_THREADS), 0, stream, ev[0], ev[1], 0,
                          (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, S_last, z_last, S_res, z_res,
                          (const bf16 *)dO, dS_out, dz_out, (bf16 *)dq, (bf16 *)dk, (bf16 *)dv, dS_in, dz_in, T);
    return hipGetLastError();
}

}  // namespace lachunk
