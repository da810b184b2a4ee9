// Forward kernel for 128-token bf16 chunks at D = 64: the blocked form of
// "Fractus-1B training optimization" (section 2, Opt 2) over the chunk's two
// 64-token blocks, computed side by side in one workgroup per group.
//
// Per block b with S_b, z_b the state before it (S_0 = S_in, S_1 = S_0 + K_0^T V_0):
//   P^T   = K_b Q_b^T, masked to j <= t (inclusive)          scores, fp32
//   den_t = sum_j P[t][j] + q_t . z_b                         (the read-after-update rule:
//   num_t = sum_j P[t][j] v_j + S_b^T q_t                      the block's own tokens are in P)
//   o_t   = num_t / den_t
//   S_out = S_1 + K_1^T V_1,  z_out = z_1 + K_1^T 1
//
// Work split (8 waves, two per SIMD): wave w owns query tile tq of block w / 4 (the
// second block's tiles in reverse, so the two waves of a SIMD carry one long and one
// short causal row range) and state tiles (key-feature tiles pt0, pt0 + 2; value tile
// ct).  Block 0 and the state are loaded first and block 1's keys and values last, so
// that block 0's outputs are computed while the rest arrives.  Three phases separated by
// two barriers:
//   A  stage block 0's K, V (and, in a one-chunk launch, block 1's); write the bf16 copy of S_0
//      and the split row of z_0
//   B  S_1 (copy + split z_1); block 0's outputs (scores, fp32 row sums, intra-block and
//      inter-block numerator, o stored); block 1's waves: the intra-block part of their outputs
//      (one-chunk launch) or the staging of block 1's K, V (sequence mode)
//   C  block 1's outputs against S_1 (the inter-block part, one-chunk launch);
//      S_out = S_1 + K_1^T V_1 stored.
// The row sums of P come straight from the fp32 accumulators (lanes hold one query
// each); P enters the numerator MFMA as a split hi + lo operand; the state copy is
// a plain bf16 operand (its term has no cancellation against the others); z_b is a
// split row so the denominator's inter-block term is exact to about 16 bits.
//
// Sequence mode (SEQ): one workgroup walks a group's n consecutive chunks in order (the
// carry across chunks of the page's section 2), the state staying in the wave's fp32
// accumulators from one chunk to the next; chunk c + 1's keys, values and queries are
// loaded into registers during chunk c (each into its staging registers as soon as they
// are free, queries into spare ones), so they arrive while c computes.  Only the first
// carry is read and the last one written.
#include "la_tile.h"
#include "la_launch.h"
#include <hip/hip_ext.h>
#include <type_traits>

namespace lachunk {

namespace {
struct Fwd2Lds {
    static constexpr int KT = 0;                  // K tiles, blocks 0 and 1
    static constexpr int VT = KT + 2 * TBYTES;    // V tiles
    static constexpr int ST = VT + 2 * TBYTES;    // S_b^T copies (bf16), b = 0, 1
    static constexpr int ZR = ST + 2 * TBYTES;    // [b][hi, lo][64] bf16 rows of z_b
    static constexpr int BYTES = ZR + 4 * 128;
    static constexpr int OS = BYTES;              // one-chunk launch: each wave's 16 x 64 tile of o
    static constexpr int BYTES_OS = OS + 8 * 2048;
    static_assert(BYTES_OS <= 160 * 1024, "LDS budget");
};
}  // namespace

template <bool SEQ, bool FM>
__device__ __forceinline__ void fwd_c128_body(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in,
    bf16 *__restrict__ o, float *__restrict__ S_out, float *__restrict__ z_out, float *__restrict__ S_res,
    float *__restrict__ z_res, int nchunk) {
    using L = Fwd2Lds;
    constexpr int D = 64, C = 128;
    constexpr uint32_t CHUNK = C * D * 2;
    __shared__ __attribute__((aligned(16))) char smem[SEQ ? L::BYTES : L::BYTES_OS];
    char *const Kt = smem + L::KT, *const Vt = smem + L::VT, *const STt = smem + L::ST, *const zrow = smem + L::ZR;

    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int blk = w >> 2;
    const int tq = blk ? 3 - (w & 3) : (w & 3);
    // state tiles: value tile ct, key-feature tiles pt0 and pt0 + 2.  The waves with ct = 0 also
    // carry z; rotating ct by pt0 puts them on different SIMDs (wave w runs on SIMD w % 4).
    const int pt0 = w >> 2, ct = (w + pt0) & 3;
    const int grp = blockIdx.x;
    const int n = SEQ ? nchunk : 1;
    // the group's tokens: n chunks of C, contiguous ([G][n C][D])
    const size_t gtok0 = (size_t)grp * n * C;
    const uint32_t seq_bytes = (uint32_t)n * CHUNK;
    const GRes qr(q + gtok0 * D, seq_bytes), kr(k + gtok0 * D, seq_bytes), vr(v + gtok0 * D, seq_bytes);
    // an absent carry is an empty range (reads give zero); the base only has to be a valid address
    const GRes sres(S_in ? (const void *)(S_in + (size_t)grp * D * D) : (const void *)S_out, S_in ? D * D * 4 : 0);
    const GRes zres(z_in ? (const void *)(z_in + (size_t)grp * D) : (const void *)z_out, z_in ? D * 4 : 0);
    // this wave's state tiles: value tile ct, key-feature tiles pt[i] = pt0 + 2i, held as
    // accumulators C[c][p] (lane: p = 16 pt[i] + r, c = 16 ct + 4g + e)
    const int pt[2] = {pt0, pt0 + 2};

    // ---- prologue: every load issued before anything waits, block 0 and the state first, so
    // that block 0's work can start while block 1's keys and values are still arriving
    bf16x8 kst0 = gload<bf16x8>(kr, tid * 16), vst0 = gload<bf16x8>(vr, tid * 16);
    bf16x8 qf[2];  // this wave's 16 queries: row t = r, k = key feature
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) qf[kc] = ldfrag_g<bf16>(qr, (64 * blk + 16 * tq) * D + 32 * kc, D, lane);
    // z is carried as the unevaluated sum zr + zc, each block's K^T 1 added exactly (two-sum):
    // it grows with every token, and the sequence backward recovers early normalisers from the
    // final one by subtraction, so z_out must be accurate to its last bit, not to the rounding
    // of thousands of additions
    // In sequence mode S is carried the same way (Sacc + Scomp): the sequence backward recovers
    // the early states from the final carry, which must then be exact beyond its rounding
    // (the remainder goes out as S_res, z_res).
    floatx4 Sacc[2], Scomp[2] = {zero4(), zero4()};
    float zr[2], zc[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        Sacc[i] = gload<floatx4>(sres, ((16 * pt[i] + r) * D + 16 * ct + 4 * g) * 4);
        zr[i] = ct == 0 ? gload<float>(zres, (16 * pt[i] + r) * 4) : 0.f;
    }
    bf16x8 kst1 = gload<bf16x8>(kr, TBYTES + tid * 16), vst1 = gload<bf16x8>(vr, TBYTES + tid * 16);
    issue_fence();
    size_t tok0 = gtok0;  // first token of the current chunk

    using Blk0 = std::integral_constant<int, 0>;
    using Blk1 = std::integral_constant<int, 1>;

    for (int c = 0; c < n; ++c) {
        // Lane-dependent offsets are derived afresh each chunk from an opaque copy of the
        // thread index: hoisted out of the loop they would all stay live across it.
        int tid_c = tid;
        if (SEQ) asm volatile("" : "+v"(tid_c));
        const int lane = tid_c & 63, r = lane & 15, g = lane >> 4;
        const TileLanes TL(lane);
        const uint32_t tr_c = TL.tr_at(ct), tr_p[2] = {TL.tr_at(pt0), TL.tr_at(pt0 + 2)}, nat_c = TL.nat_at(ct);
        const uint32_t so = stage_off(tid_c);
        // bf16 copy of S_b (row p, column c) and the split row of z_b, from the state accumulators
        auto write_state = [&](int b) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                tstore_acc(STt + b * TBYTES, nat_c, pt[i], pack4(SEQ ? Sacc[i] + Scomp[i] : Sacc[i]));
                if (ct == 0 && g == 0) {
                    bf16x2 hi, lo;
                    split_pair(zr[i] + zc[i], 0.f, hi, lo);
                    const int off = 2 * (16 * pt[i] + r);
                    *reinterpret_cast<bf16 *>(zrow + (2 * b) * 128 + off) = hi[0];
                    *reinterpret_cast<bf16 *>(zrow + (2 * b + 1) * 128 + off) = lo[0];
                }
            }
        };
        // State: S += K_b^T V_b as C[c][p] = sum_j V[j][c] K[j][p]; z += K_b^T 1
        const bf16x8 ones = ones_frag<bf16>();
        auto advance = [&](int b) {
            bf16x8 vt[2], kt[2][2];
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                vt[kc] = tfrag_tr(Vt + b * TBYTES, tr_c, kc);
#pragma unroll
                for (int i = 0; i < 2; ++i) kt[kc][i] = tfrag_tr(Kt + b * TBYTES, tr_p[i], kc);
            }
            // sequence mode: the block's K^T V in fresh accumulators, added with a two-sum
            floatx4 P[2] = {zero4(), zero4()};
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int i = 0; i < 2; ++i) mma(SEQ ? P[i] : Sacc[i], vt[kc], kt[kc][i]);
            if constexpr (SEQ) {
#pragma unroll
                for (int i = 0; i < 2; ++i) two_sum4(Sacc[i], Scomp[i], P[i]);
            }
            if (ct == 0) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    floatx4 pz = zero4();  // the block's K^T 1 (all four entries equal)
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc) mma(pz, ones, kt[kc][i]);
                    two_sum(zr[i], zc[i], pz[0]);
                }
            }
        };
        // this wave's outputs for block B (its own block), in two parts:
        //   intra : scores P^T[j][t] (lane: query t = r, key j = 16 jt + 4g + i) masked to j <= t,
        //           their fp32 row sums, and num^T[c][t] = sum_j V^T[c][j] P[t][j] (P split);
        //   finish: num^T += sum_p S_B^T[c][p] q_t[p], den = row sums + z_B . q_t, o stored.
        struct Part {
            floatx4 nm[4];
            float dsum;
        };
        auto intra = [&](auto b_tag, Part &pa) {
            constexpr int B = decltype(b_tag)::value;
            const char *Kb = Kt + B * TBYTES, *Vb = Vt + B * TBYTES;
            bf16x8 kf[4][2];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) kf[jt][kc] = jt <= tq ? tfrag(Kb, TL, jt, kc) : qf[kc];
            floatx4 sc[4];
            float dsum = 0.f;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                sc[jt] = zero4();
                if (jt <= tq) {
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc) mma(sc[jt], kf[jt][kc], qf[kc]);
                    if (jt == tq) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) sc[jt][e] = 4 * g + e <= r ? sc[jt][e] : 0.f;
                    }
                    dsum += (sc[jt][0] + sc[jt][1]) + (sc[jt][2] + sc[jt][3]);
                }
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) pa.nm[c] = zero4();
#pragma unroll
            for (int jc = 0; jc < 2; ++jc) {
                if (2 * jc <= tq) {
                    bf16x8 vf[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) vf[c] = tfrag_tr(Vb, TL.tr[c], jc);
                    const Split8 pf = split_acc(sc[2 * jc], sc[2 * jc + 1]);
#pragma unroll
                    for (int c = 0; c < 4; ++c) mma_s(pa.nm[c], vf[c], pf);
                }
            }
            pa.dsum = dsum;
        };
        // inter-block terms against the state before this block (read before it is updated)
        auto finish = [&](auto b_tag, Part &pa) {
            constexpr int B = decltype(b_tag)::value;
            const char *STb = STt + B * TBYTES, *zb = zrow + 2 * B * 128;
            bf16x8 sf[2][4], zf[2][2];
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
                for (int c = 0; c < 4; ++c) sf[kc][c] = tfrag_tr(STb, TL.tr[c], kc);
                zf[kc][0] = rowfrag(zb, lane, kc);
                zf[kc][1] = rowfrag(zb + 128, lane, kc);
            }
            floatx4 dn = zero4();
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
                for (int c = 0; c < 4; ++c) mma(pa.nm[c], sf[kc][c], qf[kc]);
                mma(dn, zf[kc][0], qf[kc]);
                mma(dn, zf[kc][1], qf[kc]);
            }
            const float inv = __builtin_amdgcn_rcpf(gsum(pa.dsum) + dn[0]);
            if constexpr (SEQ) {
                bf16 *orow = o + (tok0 + 64 * B + 16 * tq + r) * D + 4 * g;
#pragma unroll
                for (int c = 0; c < 4; ++c) store_bf16x4<false>(orow + 16 * c, pack4(pa.nm[c] * inv));
            } else {
                // the wave's 16 x 64 tile through its own LDS slab (8-byte units XOR-swizzled by row:
                // conflict-free both ways), then out as whole 128-byte rows, 16 bytes per lane
                char *slab = smem + L::OS + w * 2048;
                const int f = 2 * (r >> 1);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    *reinterpret_cast<bf16x4 *>(slab + r * 128 + 8 * ((4 * c + g) ^ f)) = pack4(pa.nm[c] * inv);
                wave_lds_sync();
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int row = 8 * i + (lane >> 3), u = lane & 7;  // 16-byte unit u of the row
                    const bf16x8 x = *reinterpret_cast<const bf16x8 *>(slab + row * 128 + 8 * ((2 * u) ^ (2 * (row >> 1))));
                    __builtin_nontemporal_store(
                        x, reinterpret_cast<bf16x8 *>(o + (tok0 + 64 * B + 16 * tq + row) * D + 8 * u));
                }
            }
        };
        auto outputs = [&](auto b_tag) {
            Part pa;
            intra(b_tag, pa);
            finish(b_tag, pa);
        };
        // Sequence mode: the next chunk's operands are loaded while this chunk computes, each
        // into its staging registers as soon as they are free (queries into spare ones).  The
        // loads are unconditional: after the last chunk their offsets lie past the buffer
        // range, which reads zeros without touching memory, and a load on every path lets
        // the compiler count outstanding loads exactly instead of draining them all.
        const uint32_t nb = (uint32_t)(c + 1) * CHUNK;
        // fused feature map: raw queries and keys in, phi applied as they are used (keys at
        // staging); the raw query fragments of this chunk are mapped here
        if constexpr (FM) {
            qf[0] = elu1_8(qf[0]);
            qf[1] = elu1_8(qf[1]);
        }
        bf16x8 nq[2];
        if (SEQ) {
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
                nq[kc] = ldfrag_g<bf16>(qr, (uint32_t)(c + 1) * C * D + (64 * blk + 16 * tq) * D + 32 * kc, D, lane);
        }

        // ---- phase A: block 0's keys and values, the S_0 copy and z_0 row; in a one-chunk launch
        // block 1's keys and values too (they arrive while block 0's are staged)
        *reinterpret_cast<bf16x8 *>(Kt + so) = FM ? elu1_8(kst0) : kst0;
        *reinterpret_cast<bf16x8 *>(Vt + so) = vst0;
        if (SEQ) {
            kst0 = gload<bf16x8>(kr, nb + tid * 16);
            vst0 = gload<bf16x8>(vr, nb + tid * 16);
        }
        write_state(0);
        if constexpr (!SEQ) {
            *reinterpret_cast<bf16x8 *>(Kt + TBYTES + so) = FM ? elu1_8(kst1) : kst1;
            *reinterpret_cast<bf16x8 *>(Vt + TBYTES + so) = vst1;
        }
        lds_barrier();

        // ---- phase B: S_1 (copy, z_1 row); block 0's outputs (their state S_0 is ready).  In a
        // one-chunk launch block 1's waves compute the intra-block part of their outputs meanwhile
        // (it needs no state); in sequence mode they stage block 1's keys and values, by now arrived.
        advance(0);
        write_state(1);
        Part pa1;
        if (blk == 0) outputs(Blk0{});
        else if (!SEQ) intra(Blk1{}, pa1);
        if constexpr (SEQ) {
            *reinterpret_cast<bf16x8 *>(Kt + TBYTES + so) = FM ? elu1_8(kst1) : kst1;
            *reinterpret_cast<bf16x8 *>(Vt + TBYTES + so) = vst1;
            kst1 = gload<bf16x8>(kr, nb + TBYTES + tid * 16);
            vst1 = gload<bf16x8>(vr, nb + TBYTES + tid * 16);
        }
        lds_barrier();

        // ---- phase C: block 1's outputs (the inter-block part against S_1 only, in a one-chunk
        // launch); the state after the chunk, S_1 + K_1^T V_1
        if (blk == 1) {
            if constexpr (SEQ) outputs(Blk1{});
            else finish(Blk1{}, pa1);
        }
        advance(1);
        if (SEQ) {
            qf[0] = nq[0];
            qf[1] = nq[1];
            tok0 += C;
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = 16 * pt[i] + r;
        const size_t so = ((size_t)grp * D + p) * D + 16 * ct + 4 * g;
        float zs, zres;
        fold(zr[i], zc[i], zs, zres);
        if constexpr (SEQ) {
            floatx4 s, res;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float a, b;
                fold(Sacc[i][e], Scomp[i][e], a, b);
                s[e] = a;
                res[e] = b;
            }
            __builtin_nontemporal_store(s, reinterpret_cast<floatx4 *>(S_out + so));
            if (S_res) __builtin_nontemporal_store(res, reinterpret_cast<floatx4 *>(S_res + so));
            if (ct == 0 && g == 0 && z_res) __builtin_nontemporal_store(zres, z_res + (size_t)grp * D + p);
        } else {
            __builtin_nontemporal_store(Sacc[i], reinterpret_cast<floatx4 *>(S_out + so));
        }
        if (ct == 0 && g == 0) __builtin_nontemporal_store(zs, z_out + (size_t)grp * D + p);
    }
}

__global__ __launch_bounds__(NTHR, 1) void la_fwd_c128_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in,
    bf16 *__restrict__ o, float *__restrict__ S_out, float *__restrict__ z_out) {
    fwd_c128_body<false, false>(q, k, v, S_in, z_in, o, S_out, z_out, nullptr, nullptr, 1);
}

// two workgroups per CU: one computes while the other waits at a barrier
__global__ __launch_bounds__(NTHR, 2) void la_seq_fwd_c128_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in,
    bf16 *__restrict__ o, float *__restrict__ S_out, float *__restrict__ z_out, float *__restrict__ S_res,
    float *__restrict__ z_res, int nchunk) {
    fwd_c128_body<true, false>(q, k, v, S_in, z_in, o, S_out, z_out, S_res, z_res, nchunk);
}

// the same with the feature map fused: q and k are the raw inputs x, the op uses elu(x) + 1
__global__ __launch_bounds__(NTHR, 2) void la_seq_fwd_c128_elu1_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in,
    bf16 *__restrict__ o, float *__restrict__ S_out, float *__restrict__ z_out, float *__restrict__ S_res,
    float *__restrict__ z_res, int nchunk) {
    fwd_c128_body<true, true>(q, k, v, S_in, z_in, o, S_out, z_out, S_res, z_res, nchunk);
}

// the one-chunk forward with the feature map fused: q and k are the raw inputs x
__global__ __launch_bounds__(NTHR, 1) void la_fwd_c128_elu1_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in,
    bf16 *__restrict__ o, float *__restrict__ S_out, float *__restrict__ z_out) {
    fwd_c128_body<false, true>(q, k, v, S_in, z_in, o, S_out, z_out, nullptr, nullptr, 1);
}

hipError_t launch_fwd_c128(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                           void *o, float *S_out, float *z_out, int G, bool elu1, hipStream_t stream,
                           const hipEvent_t ev[2]) {
    hipExtLaunchKernelGGL(elu1 ? la_fwd_c128_elu1_kernel : la_fwd_c128_kernel, dim3((unsigned)G), dim3(NTHR), 0,
                          stream, ev[0], ev[1], 0, (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, S_in, z_in,
                          (bf16 *)o, S_out, z_out);
    return hipGetLastError();
}

hipError_t launch_seq_fwd_c128(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                               void *o, float *S_out, float *z_out, float *S_res, float *z_res, int G, int nchunk,
                               bool elu1, hipStream_t stream, const hipEvent_t ev[2]) {
    hipExtLaunchKernelGGL(elu1 ? la_seq_fwd_c128_elu1_kernel : la_seq_fwd_c128_kernel, dim3((unsigned)G), dim3(NTHR),
                          0, stream, ev[0], ev[1], 0, (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, S_in, z_in,
                          (bf16 *)o, S_out, z_out, S_res, z_res, nchunk);
    return hipGetLastError();
}

}  // namespace lachunk
