// Backward kernel for 128-token bf16 chunks at D = 64: the reverse scan of
// "Fractus-1B training optimization" (section 1: the gradient of a prefix sum is a
// suffix sum) over the blocked form of section 2, Opt 2, one workgroup of 16 waves
// (four per SIMD) per group.
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
// den and rho come from fp32 accumulators (A, G are exact products of the bf16 inputs),
// so the scores never enter a second product in pass 1.  fp32 intermediates that are
// MFMA operands (S_b, dP, A inv, dN, Sh) are split hi + lo.
//
// The kernel is bound by latency at this size (one workgroup per CU, a few thousand
// dependent instructions), so the work is cut into 16 waves, four per SIMD:
//   pass 1: two waves per query tile (8 tiles: block w%8 / 4; the second block's tiles
//           reversed so each SIMD holds a long and a short causal range); half h = w / 8
//           takes key tiles 2h, 2h+1 (A, G, dP) and key-feature tiles 2h, 2h+1 (H, dq);
//           the two halves' row sums meet in LDS
//   state : one 16 x 16 tile per wave (value tile w%4, key-feature tile w/4) for S_1, Sh_0
//           and dS_in
//   pass 2: one (block, key tile, output) task per wave: dv on waves 0-7, dk on 8-15
// Phases, separated by LDS-only barriers:
//   0  stage Q, K, V, dO; split copies of S_0 and Sh_1; z_0, zh_1
//   1  S_1 (split copy, z_1); A and G of the wave's key tiles
//   2  H of the wave's key-feature tiles; partial row sums
//   3  den, rho; dP of the wave's key tiles (split, stored for dq and pass 2); inv, rho, dden
//   4  dq; Sh_0 = Sh_1 + Q_1^T dN_1 (split copy), zh_0; pass 2 of block 1 and the
//      intra-block part of pass 2 of block 0
//   5  the inter-block part of pass 2 of block 0; dS_in = Sh_0 + Q_0^T dN_0
//
// Sequence mode (SEQ): one workgroup walks a group's n consecutive chunks last to first,
// carrying the reverse state (Sh, zh) in registers from one chunk to the one before it.
// The forward state comes from the carry after the last chunk instead of per-chunk
// carries: going backwards, S_1 = S_end - K_1^T V_1 and S_0 = S_1 - K_0^T V_0 (exact
// products of the inputs, summed in fp32), and S_0 is the previous chunk's S_end.  Chunk
// c - 1's inputs are loaded into the staging registers while chunk c computes.
#include "la_tile.h"
#include "la_launch.h"
#include <hip/hip_ext.h>
#include <type_traits>

namespace lachunk {

namespace {
constexpr int W16_THREADS = 1024;

struct Bwd4Lds {
    static constexpr int QT = 0;                 // Q[2], K[2], V[2], dO[2] tiles
    static constexpr int KT = QT + 2 * TBYTES;
    static constexpr int VT = KT + 2 * TBYTES;
    static constexpr int GT = VT + 2 * TBYTES;
    // from 64 KB (addressed from base H1): split states and dP; from 128 KB (base H2): the
    // rest.  Each region's offsets from its base fit the ds instructions' 16-bit offset field.
    static constexpr int H1 = 0x10000, H2 = 0x20000;
    static constexpr int SS = GT + 2 * TBYTES;   // [b][hi, lo] split S_b; from phase 4: Sh_0 [hi, lo]
    static constexpr int DP = SS + 4 * TBYTES;   // [b][hi, lo] split dP, stored [t][j]
    static constexpr int SH1 = DP + 4 * TBYTES;  // Sh_1 [hi, lo]
    static constexpr int ZF = SH1 + 2 * TBYTES;  // [b][64] z_b fp32
    static constexpr int ZH = ZF + 2 * 64 * 4;   // [b][64] zh_b fp32
    static constexpr int INV = ZH + 2 * 64 * 4;  // [128] inv_t
    static constexpr int RHO = INV + 128 * 4;    // [128] rho_t
    static constexpr int DDR = RHO + 128 * 4;    // [hi, lo][128] dden_t bf16
    static constexpr int PS = DDR + 2 * 128 * 2; // [8 query tiles][2 halves][16 rows] (den, rho den) partials
    static constexpr int BYTES = PS + 8 * 2 * 16 * 8;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(SS == H1 && DP + 4 * TBYTES <= H1 + 0x10000 && SH1 == H2 && BYTES <= H2 + 0x10000,
                  "high regions within 64 KB of their bases");
};
}  // namespace

// S_in, z_in: the carry before the chunk (single chunk) or after the last chunk (SEQ).
// S_res, z_res (SEQ, may be NULL): the remainders of the final carry, whose exact value is
// S_in + S_res, z_in + z_res.
template <bool SEQ, bool FM>
__device__ __forceinline__ void bwd_c128_body(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in, const float *__restrict__ S_res,
    const float *__restrict__ z_res, const bf16 *__restrict__ dO,
    const float *__restrict__ dS_out, const float *__restrict__ dz_out,
    bf16 *__restrict__ dq, bf16 *__restrict__ dk, bf16 *__restrict__ dv,
    float *__restrict__ dS_in, float *__restrict__ dz_in, int nchunk) {
    using L = Bwd4Lds;
    constexpr int D = 64, C = 128;
    constexpr uint32_t CHUNK = C * D * 2;
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    float *const zf = reinterpret_cast<float *>(smem + L::ZF);
    float *const zh = reinterpret_cast<float *>(smem + L::ZH);
    float *const invs = reinterpret_cast<float *>(smem + L::INV);
    float *const rhos = reinterpret_cast<float *>(smem + L::RHO);
    bf16 *const ddr = reinterpret_cast<bf16 *>(smem + L::DDR);
    floatx2 *const psum = reinterpret_cast<floatx2 *>(smem + L::PS);
    auto tile = [&](int base, int b) -> char * { return smem + base + b * TBYTES; };
    // Tiles of the high regions, relative to their bases (paired with TL1 / TL2 offsets).  The
    // sequence loop has no registers to spare for the based offsets: there the bases are zero.
    constexpr int H1 = SEQ ? 0 : L::H1, H2 = SEQ ? 0 : L::H2;
    auto tile1 = [&](int base, int b) -> char * { return smem + base + b * TBYTES - H1; };
    auto tile2 = [&](int base, int b) -> char * { return smem + base + b * TBYTES - H2; };

    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // pass 1: query tile u (block blk, tile tq) and half h
    const int u = w & 7, h = w >> 3;
    const int blk = u >> 2;
    const int tq = blk ? 3 - (u & 3) : (u & 3);
    // state tile: value tile ct, key-feature tile pt.  The waves with ct = 0 also carry z and zh;
    // rotating ct by pt puts one of them on each SIMD (wave w runs on SIMD w % 4).
    const int pt = w >> 2, ct = (w + pt) & 3;
    const int grp = blockIdx.x;
    const int n = SEQ ? nchunk : 1;
    const size_t gtok0 = (size_t)grp * n * C;  // the group's n chunks, contiguous
    const uint32_t seq_bytes = (uint32_t)n * CHUNK;
    const GRes qr(q + gtok0 * D, seq_bytes), kr(k + gtok0 * D, seq_bytes), vr(v + gtok0 * D, seq_bytes),
        gr(dO + gtok0 * D, seq_bytes);
    const float *const dummy = dS_in;  // a valid base for an empty range
    const GRes sres(S_in ? (const void *)(S_in + (size_t)grp * D * D) : dummy, S_in ? D * D * 4 : 0);
    const GRes zres(z_in ? (const void *)(z_in + (size_t)grp * D) : dummy, z_in ? D * 4 : 0);
    const GRes shres(dS_out ? (const void *)(dS_out + (size_t)grp * D * D) : dummy, dS_out ? D * D * 4 : 0);
    const GRes zhres(dz_out ? (const void *)(dz_out + (size_t)grp * D) : dummy, dz_out ? D * 4 : 0);
    const GRes srres(S_res ? (const void *)(S_res + (size_t)grp * D * D) : dummy, S_res ? D * D * 4 : 0);
    const GRes zrres(z_res ? (const void *)(z_res + (size_t)grp * D) : dummy, z_res ? D * 4 : 0);

    // ---- prologue: every load issued before anything waits.  Thread tid stages 16 bytes of
    // Q, K, V and dO of block tid / 512.
    const int sb = tid >> 9;
    const uint32_t gso = sb * TBYTES + (tid & 511) * 16;
    bf16x8 st[4];
    auto load_stage = [&](int c) {
        const uint32_t o = (uint32_t)c * CHUNK + gso;
        st[0] = gload<bf16x8>(qr, o);
        st[1] = gload<bf16x8>(kr, o);
        st[2] = gload<bf16x8>(vr, o);
        st[3] = gload<bf16x8>(gr, o);
    };
    load_stage(n - 1);
    // state accumulators C[c][p] (lane: p = 16 pt + r, c = 16 ct + 4g + e): S and Sh
    floatx4 Sacc, Sh, zr, zhr;
    // Sequence mode: the forward state recovered from the final carry is kept as the unevaluated
    // sum (Sacc + Scomp, zr + zcomp).  Early in a long sequence the state is far smaller than the
    // final carry it is recovered from (z grows with every token), so the plain fp32 differences
    // would leave errors relative to the final carry; the compensation terms keep the rounding
    // error of every subtraction (an exact two-difference), leaving the state accurate relative
    // to itself.  They start from the final carry's remainders when those are given.
    floatx4 Scomp = zero4();
    float zcomp = 0.f;  // the four entries of z's accumulator are equal; one is carried
    {
        const uint32_t so = ((16 * pt + r) * D + 16 * ct + 4 * g) * 4;
        if (SEQ) {
            Scomp = gload<floatx4>(srres, so);
            zcomp = ct == 0 ? gload<float>(zrres, (16 * pt + r) * 4) : 0.f;
        }
        Sacc = gload<floatx4>(sres, so);
        Sh = gload<floatx4>(shres, so);
        const float a = ct == 0 ? gload<float>(zres, (16 * pt + r) * 4) : 0.f;
        const float b = ct == 0 ? gload<float>(zhres, (16 * pt + r) * 4) : 0.f;
        zr = floatx4{a, a, a, a};
        zhr = floatx4{b, b, b, b};
    }
    issue_fence();

    for (int c = n - 1; c >= 0; --c) {
        // Lane-dependent offsets are derived afresh each chunk from an opaque copy of the thread
        // index: hoisted out of the loop they would all stay live across it (and spill).
        int tid_c = tid;
        if (SEQ) asm volatile("" : "+v"(tid_c));
        const int lane = tid_c & 63, r = lane & 15, g = lane >> 4;
        const TileLanes TL(lane), TL1(lane, SEQ ? 0u : opaque_v(H1)), TL2(lane, SEQ ? 0u : opaque_v(H2));
        const uint32_t tr_c = TL.tr_at(ct), tr_p = TL.tr_at(pt);
        // small arrays past H2: per-lane byte offsets from that base
        const uint32_t g16 = TL2.base + 16 * g, g8 = TL2.base + 8 * g, r8 = TL2.base + 8 * r;
        auto f4 = [&](int off) { return *reinterpret_cast<const floatx4 *>(smem - H2 + off + g16); };
        const size_t tok0 = gtok0 + (size_t)c * C;
        // the reverse state after this chunk is nonzero unless it is the last one without dS_out
        const bool has_up = (SEQ && c < n - 1) || dS_out != nullptr;

        // ---- phase 0
        {
            const uint32_t so = sb * TBYTES + stage_off(tid_c & 511);
            // fused feature map: raw queries and keys are mapped as they are staged
            *reinterpret_cast<bf16x8 *>(smem + L::QT + so) = FM ? elu1_8(st[0]) : st[0];
            *reinterpret_cast<bf16x8 *>(smem + L::KT + so) = FM ? elu1_8(st[1]) : st[1];
            *reinterpret_cast<bf16x8 *>(smem + L::VT + so) = st[2];
            *reinterpret_cast<bf16x8 *>(smem + L::GT + so) = st[3];
        }
        // the chunk before, in flight during this one.  Unconditional: for c = 0 the offsets lie
        // past the buffer range (reads give zero, memory is not touched), and a load on every
        // path lets the compiler count outstanding loads exactly instead of draining them all.
        if (SEQ) load_stage(c - 1);
        // split copy of the wave's state tile (C[c][p] accumulator), stored [p][c] (hi, lo tiles)
        auto write_split = [&](char *hi, char *lo, const floatx4 &acc, uint32_t natc) {
            bf16x4 hh, ll;
            split4(acc, hh, ll);
            tstore_acc(hi, natc, pt, hh);
            tstore_acc(lo, natc, pt, ll);
        };
        auto write_z = [&](float *dst, const floatx4 &zz) {
            if (ct == 0 && g == 0) dst[16 * pt + r] = zz[0];
        };
        if (!SEQ) {
            write_split(tile1(L::SS, 0), tile1(L::SS, 1), Sacc, TL1.nat_at(ct));
            write_z(zf, zr);
        }
        if (has_up) write_split(tile2(L::SH1, 0), tile2(L::SH1, 1), Sh, TL2.nat_at(ct));
        write_z(zh + 64, zhr);
        lds_barrier();

        // ---- phase 1.  Forward state of block b as C[c][p] = sum_j V[j][c] K[j][p] and z: in order,
        // S_1 = S_0 + K_0^T V_0; in sequence mode backwards, S_1 = S_end - K_1^T V_1 (copy written
        // here), then S_0 = S_1 - K_0^T V_0
        const bf16x8 ones = ones_frag<bf16>();
        auto state_step = [&](int b) {
            bf16x8 vt[2], kt[2];
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                vt[kc] = tfrag_tr(tile(L::VT, b), tr_c, kc);
                kt[kc] = tfrag_tr(tile(L::KT, b), tr_p, kc);
            }
            if constexpr (SEQ) {
                // the block's K^T V and K^T 1 in fresh accumulators, then subtracted exactly
                floatx4 P = zero4(), Pz = zero4();
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) mma(P, vt[kc], kt[kc]);
                two_diff4(Sacc, Scomp, P);
                if (ct == 0) {
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc) mma(Pz, ones, kt[kc]);
                    float z0 = zr[0];
                    two_diff(z0, zcomp, Pz[0]);
                    zr[0] = z0;
                }
            } else {
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) mma(Sacc, vt[kc], kt[kc]);
                if (ct == 0) {
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc) mma(zr, ones, kt[kc]);
                }
            }
        };
        if (SEQ) {
            state_step(1);
            write_split(tile1(L::SS, 2), tile1(L::SS, 3), Sacc + Scomp, TL1.nat_at(ct));
            write_z(zf + 64, floatx4{zr[0] + zcomp, 0.f, 0.f, 0.f});
            state_step(0);
        } else {
            state_step(0);
        }
        // pass-1 operands: this wave's queries (row t = r, k = feature)
        bf16x8 qf[2], df[2];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            qf[kc] = tfrag(tile(L::QT, blk), TL, tq, kc);
            df[kc] = tfrag(tile(L::GT, blk), TL, tq, kc);
        }
        // A^T, G^T (lane: query t = r, key j = 16 (2h + jj) + 4g + i), masked to j <= t.  Key tile
        // j4 = 2h + jj lies below the query tile's diagonal (j4 < tq: no mask), on it (j4 == tq:
        // masked per element) or above it (j4 > tq: zero).  A one-chunk launch skips the products
        // of the tiles above the diagonal (uniform per wave); the sequence loop, short of
        // registers, computes every tile and masks them all.
        floatx4 aT[2], gT[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            aT[jj] = zero4();
            gT[jj] = zero4();
            const int j4 = 2 * h + jj;
            if (!SEQ && j4 > tq) continue;
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                mma(aT[jj], tfrag(tile(L::KT, blk), TL, j4, kc), qf[kc]);
                mma(gT[jj], tfrag(tile(L::VT, blk), TL, j4, kc), df[kc]);
            }
            if (SEQ || j4 == tq) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool keep = j4 < tq || (j4 == tq && 4 * g + e <= r);
                    aT[jj][e] = keep ? aT[jj][e] : 0.f;
                    gT[jj][e] = keep ? gT[jj][e] : 0.f;
                }
            }
        }
        if (SEQ) {
            write_split(tile1(L::SS, 0), tile1(L::SS, 1), Sacc + Scomp, TL1.nat_at(ct));
            write_z(zf, floatx4{zr[0] + zcomp, 0.f, 0.f, 0.f});
        } else {
            write_split(tile1(L::SS, 2), tile1(L::SS, 3), Sacc, TL1.nat_at(ct));
            write_z(zf + 64, zr);
        }
        lds_barrier();

        // ---- phase 2.  H^T[p][t] = sum_c S_b[p][c] dO[t][c] for key-feature tiles 2h, 2h+1
        // (lane: t = r, p = 16 (2h + pp) + 4g + i); partial row sums of this half
        floatx4 hT[2], zv[2];
        {
            bf16x8 sh[2][2], sl[2][2];
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    sh[pp][kc] = tfrag(tile1(L::SS, 2 * blk), TL1, 2 * h + pp, kc);
                    sl[pp][kc] = tfrag(tile1(L::SS, 2 * blk + 1), TL1, 2 * h + pp, kc);
                }
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                hT[pp] = zero4();
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    mma(hT[pp], sh[pp][kc], df[kc]);
                    mma(hT[pp], sl[pp][kc], df[kc]);
                }
            }
        }
        {
            float dpart = 0.f, rpart = 0.f;
            const bf16x8 qh = h ? qf[1] : qf[0];  // key features 32h..32h+31 of q_t
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                zv[pp] = f4(L::ZF + 4 * (64 * blk + 16 * (2 * h + pp)));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // q_t[p] for p = 16 (2h + pp) + 4g + e: k-chunk h, slot 4 pp + e
                    const float qv = (float)qh[4 * pp + e];
                    dpart += qv * zv[pp][e];
                    rpart += qv * hT[pp][e];
                }
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                if (!SEQ && 2 * h + jj > tq) continue;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dpart += aT[jj][e];
                    rpart += aT[jj][e] * gT[jj][e];
                }
            }
            const float dsum = gsum(dpart), rsum = gsum(rpart);
            if (g == 0) psum[(u * 2 + h) * 16 + r] = floatx2{dsum, rsum};
        }
        lds_barrier();

        // ---- phase 3.  Row statistics from both halves; dP for this wave's key tiles
        float inv, dden;
        {
            const floatx2 mine = *reinterpret_cast<const floatx2 *>(smem - H2 + L::PS + 8 * 16 * (u * 2 + h) + r8);
            const floatx2 other =
                *reinterpret_cast<const floatx2 *>(smem - H2 + L::PS + 8 * 16 * (u * 2 + 1 - h) + r8);
            const float den = mine[0] + other[0];
            inv = __builtin_amdgcn_rcpf(den);
            const float rho = (mine[1] + other[1]) * inv;
            dden = -rho * inv;
            // dP^T[j][t] = inv (G - rho), masked; split; stored [t][j] for dq and pass 2 (the tiles
            // above the diagonal as zeros: pass 2 reads them within its 32-query slabs)
            Split8 dps{};
            if (SEQ || 2 * h <= tq) {
                floatx4 d[2];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int j4 = 2 * h + jj;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool keep = j4 < tq || (j4 == tq && 4 * g + e <= r);
                        d[jj][e] = keep ? (gT[jj][e] - rho) * inv : 0.f;
                    }
                }
                dps = split_acc(d[0], d[1]);
            }
            tstore_frag_at(tile1(L::DP, 2 * blk), TL1, tq, h, dps.hi);
            tstore_frag_at(tile1(L::DP, 2 * blk + 1), TL1, tq, h, dps.lo);
            if (h == 0 && g == 0) {
                const int t = 64 * blk + 16 * tq + r;
                invs[t] = inv;
                rhos[t] = rho;
                bf16x2 hh, ll;
                split_pair(dden, 0.f, hh, ll);
                ddr[t] = hh[0];
                ddr[128 + t] = ll[0];
            }
        }
        lds_barrier();

        // ---- phase 4.  dq^T[p][t] = sum_j K^T[p][j] dP[t][j] + inv H^T[p][t] + dden z_b[p]
        {
            // key chunk jc (keys 32 jc .. 32 jc + 31) holds keys at or before the query tile iff
            // 2 jc <= tq (uniform); the other's dP is zero
            bf16x8 dph[2], dpl[2], ktr[2][2];
#pragma unroll
            for (int jc = 0; jc < 2; ++jc) {
                if (!SEQ && 2 * jc > tq) continue;
                dph[jc] = tfrag(tile1(L::DP, 2 * blk), TL1, tq, jc);
                dpl[jc] = tfrag(tile1(L::DP, 2 * blk + 1), TL1, tq, jc);
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) ktr[pp][jc] = tfrag_tr(tile(L::KT, blk), TL.tr_at(2 * h + pp), jc);
            }
            bf16 *dqrow = dq + (tok0 + 64 * blk + 16 * tq + r) * D + 4 * g;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                floatx4 acc = hT[pp] * inv + dden * zv[pp];
#pragma unroll
                for (int jc = 0; jc < 2; ++jc) {
                    if (!SEQ && 2 * jc > tq) continue;
                    mma(acc, ktr[pp][jc], dph[jc]);
                    mma(acc, ktr[pp][jc], dpl[jc]);
                }
                // fused feature map: the gradient of the raw query is dq phi'(x), phi' = min(1, phi)
                if constexpr (FM) acc *= elu1_grad4(lds_b64(tile(L::QT, blk) + tq * 16 * TROW + TL.nat_at(2 * h + pp)));
                if constexpr (SEQ) {
                    store_bf16x4<false>(dqrow + 16 * (2 * h + pp), pack4(acc));
                } else {
                    // staged into the S_1 copy's tile of this block (no longer read): the two
                    // halves of each row meet there, and whole rows go out in phase 5
                    tstore_acc(smem + L::SS + (2 + blk) * TBYTES, TL.nat_at(2 * h + pp), tq, pack4(acc));
                }
            }
        }
        // reverse state: Sh += Q_b^T dN_b as C[c][p] = sum_t dN[t][c] Q[t][p], zh += Q_b^T dden_b;
        // dN^T (operand rows c, k = t) is dO^T scaled by inv_t
        auto reverse = [&](int b) {
            bf16x8 xg[2], qt[2];
            floatx4 iv[2][2];
#pragma unroll
            for (int tc = 0; tc < 2; ++tc) {
                xg[tc] = tfrag_tr(tile(L::GT, b), tr_c, tc);
                qt[tc] = tfrag_tr(tile(L::QT, b), tr_p, tc);
                iv[tc][0] = f4(L::INV + 4 * (64 * b + 32 * tc));
                iv[tc][1] = f4(L::INV + 4 * (64 * b + 32 * tc + 16));
            }
#pragma unroll
            for (int tc = 0; tc < 2; ++tc) {
                const bf16x8 x = xg[tc];
                const floatx4 a0{(float)x[0] * iv[tc][0][0], (float)x[1] * iv[tc][0][1], (float)x[2] * iv[tc][0][2],
                                 (float)x[3] * iv[tc][0][3]};
                const floatx4 a1{(float)x[4] * iv[tc][1][0], (float)x[5] * iv[tc][1][1], (float)x[6] * iv[tc][1][2],
                                 (float)x[7] * iv[tc][1][3]};
                mma_s(Sh, split_acc(a0, a1), qt[tc]);
            }
            if (ct == 0) {
#pragma unroll
                for (int tc = 0; tc < 2; ++tc) {
                    // the dden row (hi, then lo) as an operand whose 16 rows are all that row
                    for (int hl = 0; hl < 2; ++hl) {
                        const char *p = smem - H2 + L::DDR + 2 * (128 * hl + 64 * b + 32 * tc) + g8;
                        mma(zhr, __builtin_shufflevector(lds_b64(p), lds_b64(p + 32), 0, 1, 2, 3, 4, 5, 6, 7), qt[tc]);
                    }
                }
            }
        };
        reverse(1);
        write_split(tile1(L::SS, 0), tile1(L::SS, 1), Sh, TL1.nat_at(ct));  // Sh_0 (the S_0 copy is no longer read)
        write_z(zh, zhr);

        // pass 2: wave w takes block (w / 4) % 2 and dv (w < 8, key tile w % 4) or dk (key tile
        // 3 - w % 4: each SIMD holds a long and a short causal range of either output);
        // accumulators dv^T[c][j] or dk^T[p][j] (lane: key j = r, column 16 x + 4g + i)
        auto pass2 = [&](auto dk_tag, auto b_tag, bool inter_phase, floatx4 (&acc)[4], bf16x8 (&kv)[2]) {
            constexpr bool DK = decltype(dk_tag)::value;
            constexpr int B = decltype(b_tag)::value;
            const int jt = DK ? 3 - (w & 3) : (w & 3);
            auto inter = [&](const char *shh, const char *shl, const TileLanes &TX) {
                if constexpr (SEQ) {
                    // half the fragments at a time: the sequence loop has fewer registers to spare
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc) {
                        bf16x8 sh[4], sl[4];
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            sh[x] = DK ? tfrag(shh, TX, x, kc) : tfrag_tr(shh, TX.tr[x], kc);
                            sl[x] = DK ? tfrag(shl, TX, x, kc) : tfrag_tr(shl, TX.tr[x], kc);
                        }
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            mma(acc[x], sh[x], kv[kc]);
                            mma(acc[x], sl[x], kv[kc]);
                        }
                    }
                    return;
                }
                bf16x8 sh[4][2], sl[4][2];
#pragma unroll
                for (int x = 0; x < 4; ++x)
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc) {
                        sh[x][kc] = DK ? tfrag(shh, TX, x, kc) : tfrag_tr(shh, TX.tr[x], kc);
                        sl[x][kc] = DK ? tfrag(shl, TX, x, kc) : tfrag_tr(shl, TX.tr[x], kc);
                    }
#pragma unroll
                for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        mma(acc[x], sh[x][kc], kv[kc]);
                        mma(acc[x], sl[x][kc], kv[kc]);
                    }
            };
            auto store = [&]() {
                bf16 *row = (DK ? dk : dv) + (tok0 + 64 * B + 16 * jt + r) * D + 4 * g;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    floatx4 y = acc[x];
                    if constexpr (DK) {
                        y += f4(L::ZH + 4 * (64 * B + 16 * x));
                        if constexpr (FM) y *= elu1_grad4(lds_b64(tile(L::KT, B) + jt * 16 * TROW + TL.nat[x]));
                    }
                    store_bf16x4<!SEQ>(row + 16 * x, pack4(y));
                }
            };
            if (inter_phase) {  // phase 5, block 0: against Sh_0
                inter(tile1(L::SS, 0), tile1(L::SS, 1), TL1);
                if constexpr (SEQ) store();
                return;
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) acc[x] = zero4();
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) kv[kc] = tfrag(tile(DK ? L::VT : L::KT, B), TL, jt, kc);
            const uint32_t tr_jt = TL1.tr_at(jt);
#pragma unroll
            for (int tc = 0; tc < 2; ++tc) {
                if (2 * tc + 1 < jt) continue;  // every query of the slab precedes the key tile
                bf16x8 xo[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) xo[x] = tfrag_tr(tile(DK ? L::QT : L::GT, B), TL.tr[x], tc);
                Split8 y;
                if constexpr (DK) {
                    // dP rows j, k = t, from the pass-1 copy
                    y = Split8{tfrag_tr(tile1(L::DP, 2 * B), tr_jt, tc), tfrag_tr(tile1(L::DP, 2 * B + 1), tr_jt, tc)};
                } else {
                    // A[t][j] inv_t recomputed (lane: j = r, t = 32 tc + 16 hh + 4g + i), masked to t >= j
                    bf16x8 qa[2][2];
                    floatx4 iv[2], at[2];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        iv[hh] = f4(L::INV + 4 * (64 * B + 32 * tc + 16 * hh));
#pragma unroll
                        for (int kc = 0; kc < 2; ++kc) qa[hh][kc] = tfrag(tile(L::QT, B), TL, 2 * tc + hh, kc);
                    }
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int t4 = 2 * tc + hh;
                        at[hh] = zero4();
#pragma unroll
                        for (int kc = 0; kc < 2; ++kc) mma(at[hh], qa[hh][kc], kv[kc]);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            at[hh][e] = (t4 > jt || (t4 == jt && 4 * g + e >= r)) ? at[hh][e] * iv[hh][e] : 0.f;
                    }
                    y = split_acc(at[0], at[1]);
                }
#pragma unroll
                for (int x = 0; x < 4; ++x) mma_s(acc[x], xo[x], y);
            }
            if (B == 1) {  // block 1 completes here, against Sh_1 = dS_out
                if (has_up) inter(tile2(L::SH1, 0), tile2(L::SH1, 1), TL2);
                if constexpr (SEQ) store();
            }
        };
        using T1 = std::integral_constant<bool, true>;
        using F1 = std::integral_constant<bool, false>;
        using B0 = std::integral_constant<int, 0>;
        using B1 = std::integral_constant<int, 1>;
        const int p2b = (w >> 2) & 1, p2dk = w >> 3;
        floatx4 acc[4];
        bf16x8 kv[2];
        if (p2dk) {
            if (p2b) pass2(T1{}, B1{}, false, acc, kv);
            else pass2(T1{}, B0{}, false, acc, kv);
        } else {
            if (p2b) pass2(F1{}, B1{}, false, acc, kv);
            else pass2(F1{}, B0{}, false, acc, kv);
        }
        lds_barrier();  // Sh_0, zh_0 visible

        // ---- phase 5
        const int tl = tid_c & 511;  // a thread's 16-byte piece of a staged tile: row tl / 8
        if constexpr (!SEQ) {
            // dq: whole 128-byte rows (8 threads per row), block sb of the staged tiles
            const bf16x8 x = *reinterpret_cast<const bf16x8 *>(smem + L::SS + (2 + sb) * TBYTES + stage_off(tl));
            __builtin_nontemporal_store(x, reinterpret_cast<bf16x8 *>(dq + (tok0 + 64 * sb + (tl >> 3)) * D + 8 * (tl & 7)));
        }
        if (p2b == 0) {
            if (p2dk) pass2(T1{}, B0{}, true, acc, kv);
            else pass2(F1{}, B0{}, true, acc, kv);
        }
        reverse(0);
        if constexpr (!SEQ) {
            // dv_b or dk_b: the wave's 16 x 64 tile through its own 2 KB slab of the dP region (no
            // longer read in this phase; 8-byte units XOR-swizzled by row, conflict-free both
            // ways), then out as whole 128-byte rows, 16 bytes per lane; no barrier, since only the
            // wave reads its slab.  dS_in straight from the accumulators, 64-byte row pieces.
            const int B = p2b, jt = p2dk ? 3 - (w & 3) : (w & 3);
            char *slab = smem + L::DP + w * 2048;
            const int f = 2 * (r >> 1);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                floatx4 y = acc[x];
                if (p2dk) {
                    y += f4(L::ZH + 4 * (64 * B + 16 * x));
                    if constexpr (FM) y *= elu1_grad4(lds_b64(tile(L::KT, B) + jt * 16 * TROW + TL.nat[x]));
                }
                *reinterpret_cast<bf16x4 *>(slab + r * 128 + 8 * ((4 * x + g) ^ f)) = pack4(y);
            }
            wave_lds_sync();
            bf16 *const out = p2dk ? dk : dv;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = 8 * i + (lane >> 3), un = lane & 7;  // 16-byte unit un of the row
                const bf16x8 x = *reinterpret_cast<const bf16x8 *>(slab + row * 128 + 8 * ((2 * un) ^ (2 * (row >> 1))));
                __builtin_nontemporal_store(
                    x, reinterpret_cast<bf16x8 *>(out + (tok0 + 64 * B + 16 * jt + row) * D + 8 * un));
            }
            const int p = 16 * pt + r;
            __builtin_nontemporal_store(Sh, reinterpret_cast<floatx4 *>(dS_in + ((size_t)grp * D + p) * D + 16 * ct + 4 * g));
        }
        // the tiles the next chunk's phase 0 writes are read up to here
        if (SEQ && c > 0) lds_barrier();
    }  // chunk loop
    {
        const int p = 16 * pt + r;
        if (SEQ)
            __builtin_nontemporal_store(Sh,
                                        reinterpret_cast<floatx4 *>(dS_in + ((size_t)grp * D + p) * D + 16 * ct + 4 * g));
        if (ct == 0 && g == 0) __builtin_nontemporal_store(zhr[0], dz_in + (size_t)grp * D + p);
    }
}

__global__ __launch_bounds__(W16_THREADS, 1) void la_bwd_c128w16_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in, const bf16 *__restrict__ dO,
    const float *__restrict__ dS_out, const float *__restrict__ dz_out,
    bf16 *__restrict__ dq, bf16 *__restrict__ dk, bf16 *__restrict__ dv,
    float *__restrict__ dS_in, float *__restrict__ dz_in) {
    bwd_c128_body<false, false>(q, k, v, S_in, z_in, nullptr, nullptr, dO, dS_out, dz_out, dq, dk, dv, dS_in, dz_in,
                                1);
}

__global__ __launch_bounds__(W16_THREADS, 1) void la_seq_bwd_c128w16_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_last, const float *__restrict__ z_last, const float *__restrict__ S_res,
    const float *__restrict__ z_res, const bf16 *__restrict__ dO,
    const float *__restrict__ dS_out, const float *__restrict__ dz_out,
    bf16 *__restrict__ dq, bf16 *__restrict__ dk, bf16 *__restrict__ dv,
    float *__restrict__ dS_in, float *__restrict__ dz_in, int nchunk) {
    bwd_c128_body<true, false>(q, k, v, S_last, z_last, S_res, z_res, dO, dS_out, dz_out, dq, dk, dv, dS_in, dz_in,
                               nchunk);
}

// the same with the feature map fused: dq and dk are the gradients of the raw inputs
__global__ __launch_bounds__(W16_THREADS, 1) void la_seq_bwd_c128w16_elu1_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_last, const float *__restrict__ z_last, const float *__restrict__ S_res,
    const float *__restrict__ z_res, const bf16 *__restrict__ dO,
    const float *__restrict__ dS_out, const float *__restrict__ dz_out,
    bf16 *__restrict__ dq, bf16 *__restrict__ dk, bf16 *__restrict__ dv,
    float *__restrict__ dS_in, float *__restrict__ dz_in, int nchunk) {
    bwd_c128_body<true, true>(q, k, v, S_last, z_last, S_res, z_res, dO, dS_out, dz_out, dq, dk, dv, dS_in, dz_in,
                              nchunk);
}

// the one-chunk backward with the feature map fused: dq and dk are the gradients of the raw inputs
__global__ __launch_bounds__(W16_THREADS, 1) void la_bwd_c128w16_elu1_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in, const bf16 *__restrict__ dO,
    const float *__restrict__ dS_out, const float *__restrict__ dz_out,
    bf16 *__restrict__ dq, bf16 *__restrict__ dk, bf16 *__restrict__ dv,
    float *__restrict__ dS_in, float *__restrict__ dz_in) {
    bwd_c128_body<false, true>(q, k, v, S_in, z_in, nullptr, nullptr, dO, dS_out, dz_out, dq, dk, dv, dS_in, dz_in,
                               1);
}

hipError_t launch_bwd_c128(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                           const void *dO, const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv,
                           float *dS_in, float *dz_in, int G, bool elu1, hipStream_t stream, const hipEvent_t ev[2]) {
    hipExtLaunchKernelGGL(elu1 ? la_bwd_c128w16_elu1_kernel : la_bwd_c128w16_kernel, dim3((unsigned)G),
                          dim3(W16_THREADS), 0, stream, ev[0], ev[1], 0, (const bf16 *)q, (const bf16 *)k,
                          (const bf16 *)v, S_in, z_in, (const bf16 *)dO, dS_out, dz_out, (bf16 *)dq, (bf16 *)dk,
                          (bf16 *)dv, dS_in, dz_in);
    return hipGetLastError();
}

hipError_t launch_seq_bwd_c128(const void *q, const void *k, const void *v, const float *S_last,
                               const float *z_last, const float *S_res, const float *z_res, const void *dO,
                               const float *dS_out, const float *dz_out, void *dq, void *dk, void *dv, float *dS_in,
                               float *dz_in, int G, int nchunk, bool elu1, hipStream_t stream,
                               const hipEvent_t ev[2]) {
    hipExtLaunchKernelGGL(elu1 ? la_seq_bwd_c128w16_elu1_kernel : la_seq_bwd_c128w16_kernel, dim3((unsigned)G),
                          dim3(W16_THREADS), 0, stream, ev[0], ev[1], 0, (const bf16 *)q, (const bf16 *)k,
                          (const bf16 *)v, S_last, z_last, S_res, z_res, (const bf16 *)dO, dS_out, dz_out, (bf16 *)dq,
                          (bf16 *)dk, (bf16 *)dv, dS_in, dz_in, nchunk);
    return hipGetLastError();
}

}  // namespace lachunk
