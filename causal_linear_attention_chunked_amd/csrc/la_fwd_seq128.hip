// Sequence forward at D = 128 (bf16): the blocked form of "Fractus-1B training optimization"
// (section 2, Opt 2) over a whole sequence of T tokens per group, the carry passed from one
// 128-token chunk to the next on chip (section 2: the carry across consecutive chunks), one
// workgroup of 8 waves per group.
//
// Per chunk, its two 64-token blocks are worked on side by side as in the 128-token D = 64
// forward: block b with S_b, z_b the state before it,
//   P^T   = K_b Q_b^T, masked to j <= t (inclusive)          scores, fp32
//   den_t = sum_j P[t][j] + q_t . z_b
//   num_t = sum_j P[t][j] v_j + S_b^T q_t,   o_t = num_t / den_t
//   S_b+1 = S_b + K_b^T V_b,   z_b+1 = z_b + K_b^T 1.
// Every wave takes part in both blocks' outputs: wave w owns value half w / 4 (64 columns) of query
// tile tq of each block (tq = w % 4 for the first half, 3 - w % 4 for the second, so that the two
// waves of a SIMD carry a long and a short causal range), and eight state tiles C[c][p]: value
// tiles 2 cp, 2 cp + 1 and key-feature tiles 4 ph .. 4 ph + 3.  The
// state and z are carried as unevaluated sums with compensation terms (each block's products
// added with a two-sum), and the final carry goes out as its nearest fp32 values and the exact
// remainders, for the sequence backward's recovery.  Three phases per chunk, two barriers:
//   A  stage block 0's K, V; the bf16 copy of S_0 and the split row of z_0
//   B  S_1 (copy, z_1 row); block 0's outputs; stage block 1's K, V
//   C  S_2 = S_1 + K_1^T V_1; block 1's outputs
// The next chunk's keys and values are loaded into the staging registers as soon as those are
// free, and a wave's queries of the next block right after its outputs are stored.  A ragged end is a masked
// block: rows past the sequence read as zero (buffer ranges) and are not stored.
// FM: q and k are raw inputs and the positive feature map elu(x) + 1 is applied inside: keys as
// they are staged (mapped keys past the end of the sequence are zero, as raw ones are: phi(0) = 1
// would count them in z), queries where they are used.
#include "la_tile.h"
#include "la_launch.h"
#include <hip/hip_ext.h>
#include <type_traits>

namespace lachunk {

namespace {
constexpr int F128_THREADS = 512;

struct Fwd128Lds {
    static constexpr int KT = 0;                 // K tiles [block][feature half]
    static constexpr int VT = KT + 4 * TBYTES;   // V tiles [block][value half]
    static constexpr int ST = VT + 4 * TBYTES;   // S_b copies (bf16) [block][p half][c half], stored [p][c]
    static constexpr int ZR = ST + 8 * TBYTES;   // [block][hi, lo][128] bf16 rows of z_b
    static constexpr int BYTES = ZR + 2 * 2 * 256;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};
}  // namespace

template <bool FM>
__device__ __forceinline__ void fwd_seq128_body(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in, bf16 *__restrict__ o,
    float *__restrict__ S_out, float *__restrict__ z_out, float *__restrict__ S_res, float *__restrict__ z_res,
    int T) {
    using L = Fwd128Lds;
    constexpr int D = 128, C = 128;
    constexpr uint32_t CHUNK = C * D * 2;  // bytes of one chunk of one token tensor
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    auto ktile = [&](int b, int f) -> char * { return smem + L::KT + (2 * b + f) * TBYTES; };
    auto vtile = [&](int b, int f) -> char * { return smem + L::VT + (2 * b + f) * TBYTES; };
    auto stile = [&](int b, int pf, int cf) -> char * { return smem + L::ST + (4 * b + 2 * pf + cf) * TBYTES; };
    char *const zrow = smem + L::ZR;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = w >> 2;
    const int tq = half ? 3 - (w & 3) : (w & 3);
    // state tiles: value tiles 2 cp, 2 cp + 1, key-feature tiles 4 ph + i.  The waves with cp = 0 also
    // carry z; rotating cp by ph puts them on SIMDs 0 and 3.
    const int ph = w >> 2, cp = (w + ph) & 3;
    const int grp = blockIdx.x;
    const int n = (T + C - 1) / C;
    const size_t gtok0 = (size_t)grp * T;
    const uint32_t seq_bytes = (uint32_t)T * D * 2;
    const GRes qr(q + gtok0 * D, seq_bytes), kr(k + gtok0 * D, seq_bytes), vr(v + gtok0 * D, seq_bytes);
    const GRes sres(S_in ? (const void *)(S_in + (size_t)grp * D * D) : (const void *)S_out, S_in ? D * D * 4 : 0);
    const GRes zres(z_in ? (const void *)(z_in + (size_t)grp * D) : (const void *)z_out, z_in ? D * 4 : 0);

    // ---- prologue: block 0's K and V, this wave's queries and the carry, then block 1's K and V.
    // Thread tid stages 16 bytes of rows tid / 16 + 32 r (r = 0, 1 for block 0; 2, 3 for block 1).
    bf16x8 kst[4], vst[4];
    auto load_kv = [&](int rr, uint32_t base) {
        kst[rr] = gload<bf16x8>(kr, base + rr * 8192 + tid * 16);
        vst[rr] = gload<bf16x8>(vr, base + rr * 8192 + tid * 16);
    };
    load_kv(0, 0);
    load_kv(1, 0);
    bf16x8 qf[4];  // this wave's 16 queries of one block: row t = r, k = key feature 32 kc ..
    auto load_q = [&](uint32_t tok, int b) {
        const int lane = tid & 63;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) qf[kc] = ldfrag_g<bf16>(qr, (tok + 64 * b + 16 * tq) * D + 32 * kc, D, lane);
    };
    load_q(0, 0);
    floatx4 Sacc[2][4], Scomp[2][4];
    float zr[4], zc[4];
    {
        const int lane = tid & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
        for (int ci = 0; ci < 2; ++ci)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = 16 * (4 * ph + i) + r;
                Sacc[ci][i] = gload<floatx4>(sres, (p * D + 16 * (2 * cp + ci) + 4 * g) * 4);
                Scomp[ci][i] = zero4();
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            zr[i] = cp == 0 ? gload<float>(zres, (16 * (4 * ph + i) + r) * 4) : 0.f;
            zc[i] = 0.f;
        }
    }
    load_kv(2, 0);
    load_kv(3, 0);
    issue_fence();
    const bf16x8 ones = ones_frag<bf16>();

    using Blk0 = std::integral_constant<int, 0>;
    using Blk1 = std::integral_constant<int, 1>;

    for (int c = 0; c < n; ++c) {
        // lane-dependent offsets derived afresh each chunk from an opaque copy of the thread index
        int tid_c = tid;
        asm volatile("" : "+v"(tid_c));
        const int lane = tid_c & 63, r = lane & 15, g = lane >> 4;
        const TileLanes TL(lane);
        const uint32_t cbase = (uint32_t)c * CHUNK;  // byte offset of this chunk
        const int nvalid = T - c * C;                // tokens of this chunk inside the sequence
        // staging slot of row tid / 16 (+ 32 r): block r / 2, row (tid / 16 + 32 r) % 64, feature half
        // (tid / 8) % 2, 16-byte unit tid % 8
        auto stage = [&](int rr) {
            const int row = (tid_c >> 4) + 32 * (rr & 1), f = (tid_c >> 3) & 1;
            const uint32_t so = stage_off(row * 8 + (tid_c & 7));
            const bool live = 64 * (rr >> 1) + row < nvalid;
            *reinterpret_cast<bf16x8 *>(ktile(rr >> 1, f) + so) = FM ? (live ? elu1_8(kst[rr]) : bf16x8{}) : kst[rr];
            *reinterpret_cast<bf16x8 *>(vtile(rr >> 1, f) + so) = vst[rr];
        };
        // bf16 copy of S_b (stored [p][c]) and the split row of z_b
        auto write_state = [&](int b) {
#pragma unroll
            for (int ci = 0; ci < 2; ++ci) {
                const int ct = 2 * cp + ci;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    tstore_acc(stile(b, ph, ct >> 2), TL.nat_at(ct & 3), i, pack4(Sacc[ci][i] + Scomp[ci][i]));
            }
            if (cp == 0 && g == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bf16x2 hi, lo;
                    split_pair(zr[i] + zc[i], 0.f, hi, lo);
                    const int off = 2 * (16 * (4 * ph + i) + r);
                    *reinterpret_cast<bf16 *>(zrow + (2 * b) * 256 + off) = hi[0];
                    *reinterpret_cast<bf16 *>(zrow + (2 * b + 1) * 256 + off) = lo[0];
                }
            }
        };
        // S += K_b^T V_b as C[c][p] = sum_j V[j][c] K[j][p], z += K_b^T 1, each block's products
        // in fresh accumulators added with a two-sum
        auto advance = [&](int b) {
            bf16x8 vt[2][2];
#pragma unroll
            for (int ci = 0; ci < 2; ++ci) {
                const int ct = 2 * cp + ci;
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) vt[ci][kc] = tfrag_tr(vtile(b, ct >> 2), TL.tr_at(ct & 3), kc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bf16x8 kt[2];
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) kt[kc] = tfrag_tr(ktile(b, ph), TL.tr[i], kc);
                floatx4 P[2] = {zero4(), zero4()};
#pragma unroll
                for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                    for (int ci = 0; ci < 2; ++ci) mma(P[ci], vt[ci][kc], kt[kc]);
#pragma unroll
                for (int ci = 0; ci < 2; ++ci) two_sum4(Sacc[ci][i], Scomp[ci][i], P[ci]);
                if (cp == 0) {
                    floatx4 pz = zero4();
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc) mma(pz, ones, kt[kc]);
                    two_sum(zr[i], zc[i], pz[0]);
                }
            }
        };
        // this wave's outputs for block B (its query tile, its value half): scores, row sums, the
        // intra-block numerator, then the inter-block terms against the state before the block; o
        // stored
        auto outputs = [&](auto b_tag) {
            constexpr int B = decltype(b_tag)::value;
            if constexpr (FM) {
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) qf[kc] = elu1_8(qf[kc]);
            }
            floatx4 sc[4];
            float dsum = 0.f;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                sc[jt] = zero4();
                if (jt <= tq) {
#pragma unroll
                    for (int kc = 0; kc < 4; ++kc) mma(sc[jt], tfrag(ktile(B, kc >> 1), TL, jt, kc & 1), qf[kc]);
                    if (jt == tq) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) sc[jt][e] = 4 * g + e <= r ? sc[jt][e] : 0.f;
                    }
                    dsum += (sc[jt][0] + sc[jt][1]) + (sc[jt][2] + sc[jt][3]);
                }
            }
            floatx4 nm[4];  // value tiles 4 half + x
#pragma unroll
            for (int x = 0; x < 4; ++x) nm[x] = zero4();
#pragma unroll
            for (int jc = 0; jc < 2; ++jc) {
                if (2 * jc <= tq) {
                    const Split8 pf = split_acc(sc[2 * jc], sc[2 * jc + 1]);
#pragma unroll
                    for (int x = 0; x < 4; ++x) mma_s(nm[x], tfrag_tr(vtile(B, half), TL.tr[x], jc), pf);
                }
            }
            floatx4 dn = zero4();
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
                for (int x = 0; x < 4; ++x) mma(nm[x], tfrag_tr(stile(B, kc >> 1, half), TL.tr[x], kc & 1), qf[kc]);
                const char *zb = zrow + 2 * B * 256 + (kc >> 1) * 128;
                mma(dn, rowfrag(zb, lane, kc & 1), qf[kc]);
                mma(dn, rowfrag(zb + 256, lane, kc & 1), qf[kc]);
            }
            const float inv = __builtin_amdgcn_rcpf(gsum(dsum) + dn[0]);
            const int trow = 64 * B + 16 * tq + r;
            if (trow < nvalid) {
                bf16 *orow = o + (gtok0 + (size_t)c * C + trow) * D + 64 * half + 4 * g;
#pragma unroll
                for (int x = 0; x < 4; ++x) store_bf16x4<false>(orow + 16 * x, pack4(nm[x] * inv));
            }
        };

        // ---- phase A: block 0's keys and values; S_0 copy and z_0 row
        stage(0);
        stage(1);
        load_kv(0, cbase + CHUNK);  // the next chunk's block 0, in flight from here
        load_kv(1, cbase + CHUNK);
        write_state(0);
        lds_barrier();

        // ---- phase B: S_1 (copy, z_1 row); block 0's outputs; block 1's keys and values
        advance(0);
        write_state(1);
        stage(2);
        stage(3);
        load_kv(2, cbase + CHUNK);
        load_kv(3, cbase + CHUNK);
        outputs(Blk0{});
        load_q((uint32_t)c * C, 1);  // block 1's queries, for phase C
        lds_barrier();

        // ---- phase C: the state after the chunk; block 1's outputs.  No barrier follows: the next
        // chunk's phase A writes block 0's tiles, the S_0 copy and z_0 row, which phase C does not read.
        advance(1);
        outputs(Blk1{});
        load_q((uint32_t)(c + 1) * C, 0);  // the next chunk's block 0 (past the end: zeros)
    }
    {
        const int lane = tid & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
        for (int ci = 0; ci < 2; ++ci)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = 16 * (4 * ph + i) + r;
                const size_t so = ((size_t)grp * D + p) * D + 16 * (2 * cp + ci) + 4 * g;
                floatx4 s, res;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float a, b;
                    fold(Sacc[ci][i][e], Scomp[ci][i][e], a, b);
                    s[e] = a;
                    res[e] = b;
                }
                *reinterpret_cast<floatx4 *>(S_out + so) = s;
                if (S_res) *reinterpret_cast<floatx4 *>(S_res + so) = res;
            }
        if (cp == 0 && g == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = 16 * (4 * ph + i) + r;
                float a, b;
                fold(zr[i], zc[i], a, b);
                z_out[(size_t)grp * D + p] = a;
                if (z_res) z_res[(size_t)grp * D + p] = b;
            }
        }
    }
}

__global__ __launch_bounds__(F128_THREADS, 1) void la_seq_fwd_d128_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in, bf16 *__restrict__ o,
    float *__restrict__ S_out, float *__restrict__ z_out, float *__restrict__ S_res, float *__restrict__ z_res,
    int T) {
    fwd_seq128_body<false>(q, k, v, S_in, z_in, o, S_out, z_out, S_res, z_res, T);
}

// the same with the feature map fused: q and k are the raw inputs x, the op uses elu(x) + 1
__global__ __launch_bounds__(F128_THREADS, 1) void la_seq_fwd_d128_elu1_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ S_in, const float *__restrict__ z_in, bf16 *__restrict__ o,
    float *__restrict__ S_out, float *__restrict__ z_out, float *__restrict__ S_res, float *__restrict__ z_res,
    int T) {
    fwd_seq128_body<true>(q, k, v, S_in, z_in, o, S_out, z_out, S_res, z_res, T);
}

hipError_t launch_seq_fwd_d128(const void *q, const void *k, const void *v, const float *S_in, const float *z_in,
                               void *o, float *S_out, float *z_out, float *S_res, float *z_res, int G, int T,
                               bool elu1, hipStream_t stream, const hipEvent_t ev[2]) {
    hipExtLaunchKernelGGL(elu1 ? la_seq_fwd_d128_elu1_kernel : la_seq_fwd_d128_kernel, dim3((unsigned)G),
                          dim3(F128_THREADS), 0, stream, ev[0], ev[1], 0,
                          (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, S_in, z_in, (bf16 *)o, S_out, z_out,
                          S_res, z_res, T);
    return hipGetLastError();
}

}  // namespace lachunk
