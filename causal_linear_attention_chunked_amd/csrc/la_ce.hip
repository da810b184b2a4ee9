// Cross-entropy over a tied output head ("Fractus-1B training optimization", section 1,
// Bottleneck #3, and section 2, Opt 3: chunked, checkpointed cross-entropy).
//
//   logit_iv = h_i . W_v,  lse_i = log sum_v exp(logit_iv),  loss = (1/N) sum_i (lse_i - logit_{i,t_i})
//   P_iv = (g/N) (exp(logit_iv - lse_i) - [v = t_i]),  dh = P W,  dW = P^T h
//
// Every product is one MFMA GEMM mainloop (bf16 operands, fp32 accumulators): a 128 x 128
// output tile per workgroup of four waves (64 x 64 each, 16 accumulator tiles), the operands
// staged 64 k at a time into two LDS buffers of swizzled 64 x 64 tiles (csrc/la_tile.h) while
// the next k-step's loads are in flight.  An operand is read from LDS with the natural fragment
// read when it is stored k-contiguous and with the transposed read when it is stored k-major, so
// no operand is ever transposed in memory.  Operand rows past the end read as zero (buffer
// ranges).  The epilogues:
//   forward: the tile's logits never leave registers: per token, the maximum and the sum of
//            exponentials over the tile's 128 classes (combined over the two waves in LDS) go to
//            a partials array, and the target's logit where it falls in the tile; a second kernel
//            combines each token's partials into lse (16 threads per token), a third takes the
//            mean loss in a fixed order (deterministic);
//   backward: the logits are recomputed (the checkpoint) and P is written in bf16, one chunk of
//            tokens at a time (the chunk's P is the transient of the pages' chunked form);
//            dW = P^T h (output tiles stored, or added for the chunks after the first) and
//            dh = P W, split over the vocabulary into partial sums that a last kernel adds.
#include "la_tile.h"
#include "la_launch.h"
#include <hip/hip_ext.h>

namespace lachunk {

namespace {
constexpr int CE_THREADS = 256;
constexpr int CT = 128;  // output tile edge
constexpr int CK = 64;   // k per stage

// Offsets (bytes) of one stage's four tiles: A rows 0-63, 64-127, then B likewise.
__device__ __forceinline__ char *stage_tile(char *smem, int stage, int op, int u) {
    return smem + ((stage * 2 + op) * 2 + u) * TBYTES;
}

struct Operand {
    GRes g;
    uint32_t ld;   // elements between consecutive storage rows
    bool kmajor;   // stored [k][row] (row contiguous) instead of [row][k]
};

// The 128 x 128 fp32 tile C[m][n] = sum_k A[m][k] B[n][k] over k in [k0, k1) (multiples of 64),
// m from row m0 of A, n from row n0 of B.  Wave w holds rows 64 (w & 1).. of m and 64 (w >> 1)..
// of n: acc[i][j] is the 16 x 16 tile (m-tile i, n-tile j), lane (r, g) holding
// C[m = 16 i + 4 g + e][n = 16 j + r].
template <bool AKM, bool BKM>
__device__ __forceinline__ void gemm_tile(char *smem, const Operand &A, const Operand &B, uint32_t m0, uint32_t n0,
                                          uint32_t k0, uint32_t k1, floatx4 (&acc)[4][4]) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w & 1, wn = w >> 1;
    const TileLanes TL(lane);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = zero4();
    // thread tid stages 16 bytes of storage rows tid / 8 and tid / 8 + 32 of each 64 x 64 tile
    const int srow = tid >> 3, sunit = tid & 7;
    typedef bf16x8 Stage[2][2][2];  // [operand][tile][half]
    auto load = [&](Stage &st, uint32_t kk) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int hv = 0; hv < 2; ++hv) {
                const uint32_t row = srow + 32 * hv;
                const uint32_t oa = AKM ? (kk + row) * A.ld + m0 + 64 * u + 8 * sunit
                                        : (m0 + 64 * u + row) * A.ld + kk + 8 * sunit;
                const uint32_t ob = BKM ? (kk + row) * B.ld + n0 + 64 * u + 8 * sunit
                                        : (n0 + 64 * u + row) * B.ld + kk + 8 * sunit;
                st[0][u][hv] = gload<bf16x8>(A.g, oa * 2);
                st[1][u][hv] = gload<bf16x8>(B.g, ob * 2);
            }
    };
    auto store = [&](const Stage &st, int stage) {
#pragma unroll
        for (int op = 0; op < 2; ++op)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int hv = 0; hv < 2; ++hv)
                    *reinterpret_cast<bf16x8 *>(stage_tile(smem, stage, op, u) + stage_off(tid + 256 * hv)) =
                        st[op][u][hv];
    };
    auto compute = [&](int stage) {
        const char *At = stage_tile(smem, stage, 0, wm), *Bt = stage_tile(smem, stage, 1, wn);
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                af[i] = AKM ? tfrag_tr(At, TL.tr[i], kc) : tfrag(At, TL, i, kc);
                bfr[i] = BKM ? tfrag_tr(Bt, TL.tr[i], kc) : tfrag(Bt, TL, i, kc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) mma(acc[i][j], af[i], bfr[j]);
        }
    };
    // One register stage: the next k-step's loads are issued before this one's products and
    // stored after them.  Measured and rejected: two stages a full k-step ahead (more registers,
    // slower), A fragments read one at a time (less overlap, slower), one 16-byte read per
    // fragment in the contiguous k order for k-contiguous operands (slower).
    const int nk = (int)((k1 - k0) / CK);
    Stage r0;
    load(r0, k0);
    store(r0, 0);
    lds_barrier();
    for (int ks = 0; ks < nk; ++ks) {
        const bool more = ks + 1 < nk;
        if (more) load(r0, k0 + (uint32_t)(ks + 1) * CK);
        compute(ks & 1);
        if (more) store(r0, (ks & 1) ^ 1);
        lds_barrier();
    }
}

// max over the four lane groups (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float gmax(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Workgroups are dealt to the eight XCDs in turn (workgroup b to XCD b % 8), each XCD with its own
// L2.  The tile order is remapped so that each XCD takes one contiguous range of logical tiles:
// tiles that share an operand are numbered consecutively, so they run on one XCD and that
// operand is fetched into one L2 instead of several.
__device__ __forceinline__ uint32_t xcd_tile(uint32_t b, uint32_t total) {
    const uint32_t per = total / 8, rem = total % 8, x = b % 8, k = b / 8;
    return x < rem ? x * (per + 1) + k : rem * (per + 1) + (x - rem) * per + k;
}

constexpr float LOG2E = 1.4426950408889634f;
__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * LOG2E); }
}  // namespace

// Forward tiles: one workgroup per (class tile, token tile).  The A operand is W (rows = classes), B is
// h (rows = tokens), both k-contiguous.  part[vt][t] = (max, sum exp(logit - max)) over the tile's
// classes, tl[t] = logit of token t's target (written by the one lane that holds it).
__global__ __launch_bounds__(CE_THREADS, 2) void la_ce_fwd_kernel(
    const bf16 *__restrict__ h, const bf16 *__restrict__ W, const int *__restrict__ targets,
    floatx2 *__restrict__ part, float *__restrict__ tl, int N, int d, int V, int Npad) {
    __shared__ __attribute__((aligned(16))) char smem[8 * TBYTES];
    // logical tile: the token tiles of one class tile consecutively (they share its rows of W)
    const uint32_t ntt = (uint32_t)Npad / CT;
    const uint32_t L = xcd_tile(blockIdx.x, gridDim.x), vt = L / ntt;
    const uint32_t v0 = vt * CT, t0 = (L % ntt) * CT;
    const Operand A{GRes(W, (uint32_t)V * d * 2), (uint32_t)d, false};
    const Operand B{GRes(h, (uint32_t)N * d * 2), (uint32_t)d, false};
    floatx4 acc[4][4];
    gemm_tile<false, false>(smem, A, B, v0, t0, 0, (uint32_t)d, acc);

    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w & 1, wn = w >> 1;
    floatx2 *const xch = reinterpret_cast<floatx2 *>(smem);  // [2 wm][128 tokens]
    const GRes tres(targets, (uint32_t)N * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int tloc = 64 * wn + 16 * j + r;
        const int t = (int)t0 + tloc;
        const int tgt = gload<int>(tres, (uint32_t)t * 4);
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int vv = (int)v0 + 64 * wm + 16 * i + 4 * g + e;
                if (vv < V) mx = fmaxf(mx, acc[i][j][e]);
                if (vv == tgt && t < N) tl[t] = acc[i][j][e];
            }
        mx = gmax(mx);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int vv = (int)v0 + 64 * wm + 16 * i + 4 * g + e;
                s += vv < V ? exp_f(acc[i][j][e] - mx) : 0.f;
            }
        s = gsum(s);
        if (g == 0) xch[wm * CT + tloc] = floatx2{mx, s};
    }
    lds_barrier();
    if (tid < CT) {
        const floatx2 a = xch[tid], b = xch[CT + tid];
        const float m = fmaxf(a[0], b[0]);
        // a tile's classes may all lie past V only if V <= v0, which the grid excludes
        const float s = a[1] * exp_f(a[0] - m) + b[1] * exp_f(b[0] - m);
        part[(size_t)vt * Npad + t0 + tid] = floatx2{m, s};
    }
}

// lse_t = max + log(sum over the class tiles' partials), nll_t = lse_t - tl_t: 16 tokens per
// workgroup, 16 threads per token each folding every 16th tile, then merged in a fixed order.
__global__ __launch_bounds__(256) void la_ce_lse_kernel(const floatx2 *__restrict__ part, const float *__restrict__ tl,
                                                       float *__restrict__ lse, float *__restrict__ nll, int N,
                                                       int Npad, int nvt) {
    const int t = blockIdx.x * 16 + (threadIdx.x >> 4), sub = threadIdx.x & 15;
    float m = -INFINITY, s = 0.f;
    if (t < N) {
        for (int vt = sub; vt < nvt; vt += 16) {
            const floatx2 p = part[(size_t)vt * Npad + t];
            const float mm = fmaxf(m, p[0]);
            s = s * exp_f(m - mm) + p[1] * exp_f(p[0] - mm);
            m = mm;
        }
    }
#pragma unroll
    for (int k = 1; k < 16; k <<= 1) {  // butterfly over the 16 threads of the token
        const float m2 = __shfl_xor(m, k), s2 = __shfl_xor(s, k);
        const float mm = fmaxf(m, m2);
        s = (m == -INFINITY ? 0.f : s * exp_f(m - mm)) + (m2 == -INFINITY ? 0.f : s2 * exp_f(m2 - mm));
        m = mm;
    }
    if (t < N && sub == 0) {
        const float l = m + __logf(s);
        lse[t] = l;
        nll[t] = l - tl[t];
    }
}

// One workgroup: loss = mean of nll, summed in a fixed order.
__global__ __launch_bounds__(1024, 1) void la_ce_mean_kernel(const float *__restrict__ nll, float *__restrict__ loss,
                                                            int N) {
    __shared__ float red[1024];
    float acc = 0.f;
    for (int t = threadIdx.x; t < N; t += 1024) acc += nll[t];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int k = 512; k > 0; k >>= 1) {
        if ((int)threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
        __syncthreads();
    }
    if (threadIdx.x == 0) *loss = red[0] / (float)N;
}

// Backward P tiles for the tokens [c0, c0 + Nc): the logits recomputed, P = scale (softmax - onehot)
// in bf16 at P[t - c0][v] (pitch Vpad); classes past V and tokens past the chunk get 0.
__global__ __launch_bounds__(CE_THREADS, 2) void la_ce_p_kernel(
    const bf16 *__restrict__ h, const bf16 *__restrict__ W, const int *__restrict__ targets,
    const float *__restrict__ lse, const float *__restrict__ dloss, bf16 *__restrict__ P, int c0, int Nc, int N,
    int d, int V, int Vpad) {
    __shared__ __attribute__((aligned(16))) char smem[8 * TBYTES];
    const uint32_t ntt = (uint32_t)(Nc + CT - 1) / CT;
    const uint32_t L = xcd_tile(blockIdx.x, gridDim.x);
    const uint32_t v0 = (L / ntt) * CT, t0 = (L % ntt) * CT;
    const Operand A{GRes(W, (uint32_t)V * d * 2), (uint32_t)d, false};
    const Operand B{GRes(h + (size_t)c0 * d, (uint32_t)Nc * d * 2), (uint32_t)d, false};
    floatx4 acc[4][4];
    gemm_tile<false, false>(smem, A, B, v0, t0, 0, (uint32_t)d, acc);

    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w & 1, wn = w >> 1;
    const float scale = (dloss ? *dloss : 1.f) / (float)N;
    const GRes tres(targets + c0, (uint32_t)Nc * 4), lres(lse + c0, (uint32_t)Nc * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int tloc = (int)t0 + 64 * wn + 16 * j + r;  // token within the chunk
        const int tgt = gload<int>(tres, (uint32_t)tloc * 4);
        const float l = gload<float>(lres, (uint32_t)tloc * 4);
        const bool live = tloc < Nc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int vb = (int)v0 + 64 * wm + 16 * i + 4 * g;
            floatx4 p;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int vv = vb + e;
                const float x = exp_f(acc[i][j][e] - l) - (vv == tgt ? 1.f : 0.f);
                p[e] = (live && vv < V) ? x * scale : 0.f;
            }
            *reinterpret_cast<bf16x4 *>(P + (size_t)tloc * Vpad + vb) = pack4(p);
        }
    }
}

// dW tiles: C[m = feature][n = class] = sum_t h[t][m] P[t][n] over the chunk's (padded) tokens;
// both operands k-major.  Stored as dW[n][m] (fp32), or added to it (accumulate).
__global__ __launch_bounds__(CE_THREADS, 2) void la_ce_dw_kernel(const bf16 *__restrict__ h,
                                                                 const bf16 *__restrict__ P, float *__restrict__ dW,
                                                                 int c0, int Nc, int Ncpad, int d, int V, int Vpad,
                                                                 int accumulate) {
    __shared__ __attribute__((aligned(16))) char smem[8 * TBYTES];
    // the feature tiles of one class tile consecutively (they share its columns of P)
    const uint32_t nft = (uint32_t)d / CT;
    const uint32_t L = xcd_tile(blockIdx.x, gridDim.x);
    const uint32_t f0 = (L % nft) * CT, v0 = (L / nft) * CT;
    const Operand A{GRes(h + (size_t)c0 * d, (uint32_t)Nc * d * 2), (uint32_t)d, true};
    const Operand B{GRes(P, (uint32_t)Ncpad * Vpad * 2), (uint32_t)Vpad, true};
    floatx4 acc[4][4];
    gemm_tile<true, true>(smem, A, B, f0, v0, 0, (uint32_t)Ncpad, acc);

    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w & 1, wn = w >> 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int vv = (int)v0 + 64 * wn + 16 * j + r;
        if (vv >= V) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            floatx4 *dst = reinterpret_cast<floatx4 *>(dW + (size_t)vv * d + f0 + 64 * wm + 16 * i + 4 * g);
            *dst = accumulate ? *dst + acc[i][j] : acc[i][j];
        }
    }
}

// dh partial tiles: C[m = feature][n = token] = sum_v W[v][m] P[t][v] over classes [k0, k1) of split
// blockIdx.z; A = W k-major, B = P k-contiguous.  Stored to part[z][t][m] (fp32).
__global__ __launch_bounds__(CE_THREADS, 2) void la_ce_dh_kernel(const bf16 *__restrict__ W,
                                                                 const bf16 *__restrict__ P, float *__restrict__ part,
                                                                 int Ncpad, int d, int V, int Vpad, int kper) {
    __shared__ __attribute__((aligned(16))) char smem[8 * TBYTES];
    // split slowest, then token tile, feature tile fastest: consecutive tiles share P's rows of the
    // split, and the tiles of one split share its rows of W
    const uint32_t nft = (uint32_t)d / CT, ntt = (uint32_t)Ncpad / CT;
    const uint32_t L = xcd_tile(blockIdx.x, gridDim.x), z = L / (nft * ntt), rest = L % (nft * ntt);
    const uint32_t f0 = (rest % nft) * CT, t0 = (rest / nft) * CT;
    const uint32_t k0 = z * (uint32_t)kper;
    const uint32_t k1 = k0 + (uint32_t)kper < (uint32_t)Vpad ? k0 + (uint32_t)kper : (uint32_t)Vpad;
    const Operand A{GRes(W, (uint32_t)V * d * 2), (uint32_t)d, true};
    const Operand B{GRes(P, (uint32_t)Ncpad * Vpad * 2), (uint32_t)Vpad, false};
    floatx4 acc[4][4];
    gemm_tile<true, false>(smem, A, B, f0, t0, k0, k1, acc);

    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w & 1, wn = w >> 1;
    float *base = part + (size_t)z * Ncpad * d;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = (int)t0 + 64 * wn + 16 * j + r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<floatx4 *>(base + (size_t)t * d + f0 + 64 * wm + 16 * i + 4 * g) = acc[i][j];
    }
}

// dh[c0 + t][m] = sum over the splits, in order, rounded to bf16 (four features per thread).
__global__ __launch_bounds__(256) void la_ce_dh_reduce_kernel(const float *__restrict__ part, bf16 *__restrict__ dh,
                                                              int c0, int Nc, int Ncpad, int d, int nsplit) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // index of four features
    const size_t n4 = (size_t)Nc * d / 4;
    if (i >= n4) return;
    floatx4 s = zero4();
    for (int z = 0; z < nsplit; ++z) s += reinterpret_cast<const floatx4 *>(part + (size_t)z * Ncpad * d)[i];
    *reinterpret_cast<bf16x4 *>(dh + (size_t)c0 * d + 4 * i) = pack4(s);
}

// ---------------------------------------------------------------- host side

CeShape ce_shape(int N, int d, int V, int ce_chunk) {
    CeShape s;
    s.Npad = (N + CT - 1) / CT * CT;
    s.Vpad = (V + CT - 1) / CT * CT;
    s.nvt = s.Vpad / CT;
    s.chunk = ce_chunk < 1 || ce_chunk > N ? N : ce_chunk;
    s.chunk_pad = (s.chunk + CT - 1) / CT * CT;
    // dh split over the vocabulary: enough workgroups to fill the chip, whole k-steps per split
    const int tiles = (d / CT) * (s.chunk_pad / CT);
    int nsplit = (512 + tiles - 1) / tiles;
    if (nsplit > s.Vpad / CK) nsplit = s.Vpad / CK;
    s.kper = ((s.Vpad + nsplit - 1) / nsplit + CK - 1) / CK * CK;
    s.nsplit = (s.Vpad + s.kper - 1) / s.kper;
    s.fwd_bytes = (size_t)s.nvt * s.Npad * 8 + (size_t)s.Npad * 8;  // partials, target logits, nll
    s.p_bytes = (size_t)s.chunk_pad * s.Vpad * 2;
    s.bwd_bytes = s.p_bytes + (size_t)s.nsplit * s.chunk_pad * d * 4;
    s.ws_bytes = s.fwd_bytes > s.bwd_bytes ? s.fwd_bytes : s.bwd_bytes;
    return s;
}

hipError_t launch_ce_fwd(const void *h, const void *W, const int *targets, float *loss, float *lse, void *ws, int N,
                         int d, int V, hipStream_t stream, const hipEvent_t ev[2]) {
    const CeShape s = ce_shape(N, d, V, N);
    floatx2 *part = reinterpret_cast<floatx2 *>(ws);
    float *tl = reinterpret_cast<float *>(static_cast<char *>(ws) + (size_t)s.nvt * s.Npad * 8);
    float *nll = tl + s.Npad;
    hipExtLaunchKernelGGL(la_ce_fwd_kernel, dim3(s.nvt * (s.Npad / CT)), dim3(CE_THREADS), 0, stream, ev[0], nullptr,
                          0, (const bf16 *)h, (const bf16 *)W, targets, part, tl, N, d, V, s.Npad);
    hipExtLaunchKernelGGL(la_ce_lse_kernel, dim3((N + 15) / 16), dim3(256), 0, stream, nullptr, nullptr, 0,
                          (const floatx2 *)part, (const float *)tl, lse, nll, N, s.Npad, s.nvt);
    hipExtLaunchKernelGGL(la_ce_mean_kernel, dim3(1), dim3(1024), 0, stream, nullptr, ev[1], 0, (const float *)nll,
                          loss, N);
    return hipGetLastError();
}

hipError_t launch_ce_bwd(const void *h, const void *W, const int *targets, const float *lse, const float *dloss,
                         void *dh, float *dW, void *ws, int N, int d, int V, int ce_chunk, hipStream_t stream,
                         const hipEvent_t ev[2]) {
    const CeShape s = ce_shape(N, d, V, ce_chunk);
    bf16 *P = static_cast<bf16 *>(ws);
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + s.p_bytes);
    for (int c0 = 0; c0 < N; c0 += s.chunk) {
        const int Nc = N - c0 < s.chunk ? N - c0 : s.chunk;
        const int Ncpad = (Nc + CT - 1) / CT * CT;
        const bool first = c0 == 0, last = c0 + s.chunk >= N;
        hipExtLaunchKernelGGL(la_ce_p_kernel, dim3(s.nvt * (Ncpad / CT)), dim3(CE_THREADS), 0, stream,
                              first ? ev[0] : nullptr, nullptr, 0, (const bf16 *)h, (const bf16 *)W, targets, lse,
                              dloss, P, c0, Nc, N, d, V, s.Vpad);
        hipExtLaunchKernelGGL(la_ce_dh_kernel, dim3((d / CT) * (Ncpad / CT) * s.nsplit), dim3(CE_THREADS), 0, stream,
                              nullptr, nullptr, 0, (const bf16 *)W, (const bf16 *)P, part, Ncpad, d, V, s.Vpad,
                              s.kper);
        const size_t n4 = (size_t)Nc * d / 4;
        hipExtLaunchKernelGGL(la_ce_dh_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                              nullptr, nullptr, 0, (const float *)part, (bf16 *)dh, c0, Nc, Ncpad, d, s.nsplit);
        hipExtLaunchKernelGGL(la_ce_dw_kernel, dim3((d / CT) * s.nvt), dim3(CE_THREADS), 0, stream, nullptr,
                              last ? ev[1] : nullptr, 0, (const bf16 *)h, (const bf16 *)P, dW, c0, Nc, Ncpad, d, V,
                              s.Vpad, first ? 0 : 1);
    }
    return hipGetLastError();
}

}  // namespace lachunk
