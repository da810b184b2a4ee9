// Cross-entropy over a tied output head ("Fractus-1B training optimization", section 1,
// Bottleneck #3, and section 2, Opt 3: chunked, checkpointed cross-entropy).
//
//   logit_iv = h_i . W_v,  lse_i = log sum_v exp(logit_iv),  loss = (1/N) sum_i (lse_i - logit_{i,t_i})
//   P_iv = (g/N) (exp(logit_iv - lse_i) - [v = t_i]),  dh = P W,  dW = P^T h
//
// Every product is one MFMA GEMM mainloop (bf16 operands, fp32 accumulators): 256 x 128 output
// tiles over eight waves (64 x 64 each, 16 accumulator tiles), persistent workgroups (one per
// CU) each walking a run of tiles, the operands loaded 64 k at a time straight from global memory
// into three LDS stages (buffer loads that write LDS), two k-steps ahead of the products, across
// tile boundaries.  The loads fill the swizzled 64 x 64 tile layout
// of csrc/la_tile.h: each load instruction writes 1 KB of consecutive LDS (eight tile rows), so
// every lane fetches the 16 bytes that belong in its slot.  An operand is read from LDS with the
// natural fragment read when it is stored k-contiguous and with the transposed read when it is
// stored k-major, so no operand is ever transposed in memory.  Operand rows past the end of an
// operand read as zero (buffer ranges), or, for a k-major operand whose rows end inside its
// storage rows, as values that only reach output rows that are not stored.  The epilogues:
//   forward: the tile's logits never leave registers: per token, the maximum and the sum of
//            exponentials over the tile's 256 classes (combined over the four waves in LDS) go to
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
#include <atomic>

namespace lachunk {

namespace {
constexpr int CE_THREADS = 512;  // eight waves
constexpr int MT = CE_MT;        // output tile rows (the A operand's)
constexpr int NT = CE_NT;        // output tile columns (the B operand's)
constexpr int CK = CE_CK;        // k per stage
constexpr int STAGE = (MT + NT) / 64 * TBYTES;  // one stage: A tiles 0-3, then B tiles 0-1 (48 KB)

typedef int int4v __attribute__((ext_vector_type(4)));
typedef uint32_t uint2v __attribute__((ext_vector_type(2)));
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Buffer descriptor of `bytes` bytes at `base` as four dwords (the layout and flags of GRes):
// reads at offsets past the range return zero and touch no memory.
__device__ __forceinline__ int4v rsrc4(const void *base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    return int4v{(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

struct Operand {
    int4v rs;      // buffer descriptor (uniform)
    uint32_t ld;   // elements between consecutive storage rows
    bool kmajor;   // stored [k][row] (row contiguous) instead of [row][k]
};

// Load into LDS: each lane's 16 bytes at voff go to LDS byte lds + 16 x lane; lds is
// uniform (M0).  Issued as assembly, so the compiler neither counts them nor orders LDS reads
// after them: the main loop waits for them itself (vmcnt) and a barrier publishes them.  Loads
// the compiler does not know of can only make its own waits for its own loads stricter.
// Nor does the compiler look inside assembly for hazards: a VALU write of an SGPR (a v_readlane
// restoring a spilled descriptor, say) needs five wait states before a vector memory instruction
// reads that SGPR.  The build compiles this file to assembly and refuses a library in which such
// a write comes closer than that to one of these loads (asm_check.py).
__device__ __forceinline__ void lds_load16(const int4v &rs, const void *lds, uint32_t voff) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rs), "{m0}"((uint32_t)(size_t)(lds_void *)lds)
                 : "memory");
}

// The same for one dword per lane: lane l's 4 bytes at voff go to LDS byte lds + 4 x lane.
__device__ __forceinline__ void lds_load4(const int4v &rs, const void *lds, uint32_t voff) {
    asm volatile("buffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rs), "{m0}"((uint32_t)(size_t)(lds_void *)lds)
                 : "memory");
}

// s_waitcnt vmcnt(n) lgkmcnt(0) (expcnt untouched), n < 16
template <int n>
__device__ __forceinline__ void wait_vm_lgkm() {
    static_assert(n >= 0 && n < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0070 | n);
}

// An output tile: rows m0.. of A, n0.. of B, k-steps k0 .. k0 + 64 nk.
struct TileRange {
    uint32_t m0, n0, k0;
    int nk;
};

// The workgroup's logical tiles.  Workgroups are dealt to the eight XCDs in turn (workgroup b to
// XCD b % 8, the grid a multiple of 8), each XCD with its own L2.  The T tiles are cut into eight
// contiguous ranges, one per XCD, and the XCD's workgroups take its tiles in turn: the tiles in
// flight on one XCD at a time are consecutive, and consecutive tiles share an operand, which is
// then fetched into one L2 instead of several.
struct TileWalk {
    uint32_t first, stride, count;
    __device__ __forceinline__ explicit TileWalk(uint32_t T) {
        const uint32_t b = blockIdx.x, x = b % 8, k = b / 8, gx = gridDim.x / 8;
        const uint32_t per = T / 8, rem = T % 8;
        const uint32_t start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
        const uint32_t cnt = per + (x < rem ? 1u : 0u);
        first = start + k;
        stride = gx;
        count = cnt > k ? (cnt - k + gx - 1) / gx : 0u;
    }
    __device__ __forceinline__ uint32_t operator[](uint32_t j) const { return first + j * stride; }
};

// Persistent GEMM over the workgroup's tiles: for each 256 x 128 tile, C[m][n] = sum_k A[m][k]
// B[n][k], handed to epi(L, acc) when its last k-step is done.  Wave w holds rows 64 (w & 3).. of m
// and 64 (w >> 2).. of n: acc[i][j] is the 16 x 16 tile (m-tile i, n-tile j), lane (r, g) holding
// C[m = 16 i + 4 g + e][n = 16 j + r].  s0, s1, s2: the three stages, separate LDS arrays.
//
// Pipeline: the k-steps of all the workgroup's tiles form one stream; step g is loaded into
// s[g % 3] two steps ahead, so the next tile's first loads are in flight during the current
// tile's last products and its epilogue.  Each step waits for the wave's own loads of the step
// (vmcnt(6): the six of the next step, always issued after them, may stay in flight; after an
// epilogue its stores and loads are newer still, so the wait then also covers some of them) and
// for its LDS reads, then a barrier: every wave's loads of the step have landed and every wave is
// done reading the stage the step after next is loaded into; then the products, with the loads
// of the step after next issued behind them, half after each k-chunk.  The loads past the end of
// the stream are issued at an offset past every buffer range (no memory is read), so that every
// step has the same loads in flight.
// pre(L), when given, runs right after the barrier of tile L's next-to-last k-step (every tile has
// at least two): loads it issues into LDS there (lds_load4) are complete and visible when the
// tile's epilogue runs, behind the next step's wait and barrier, so the epilogue never waits on
// memory (a load of its own would wait for every load in flight, the stages' too).
struct NoPre {
    __device__ __forceinline__ void operator()(uint32_t) const {}
};
template <bool AKM, bool BKM, class TileF, class EpiF, class PreF = NoPre>
__device__ __forceinline__ void gemm_tiles(char *s0, char *s1, char *s2, const Operand &A, const Operand &B,
                                           const TileWalk &walk, TileF tile_at, EpiF epi, PreF pre = PreF{}) {
    if (walk.count == 0) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w & 3, wn = w >> 2;
    const TileLanes TL(lane);
    int S = 0;  // k-steps of all the workgroup's tiles
    for (uint32_t j = 0; j < walk.count; ++j) S += tile_at(walk[j]).nk;

    // Load instruction i of wave w writes rows 8w..8w+7 of tile i (A tiles 0-3, then B tiles 0-1);
    // lane l lands in storage row y = 8w + l / 8, 16-byte slot l % 8, which holds the row's logical
    // 16-byte unit (l % 8) ^ (swz(y) / 2).  Element offsets of the lane's units at k = 0 of the
    // tile the load cursor is in:
    const int y = 8 * w + (lane >> 3);
    const int uu = (lane & 7) ^ ((y ^ (y >> 1)) & 7);
    uint32_t ij = 0;  // load cursor: tile ij (itr), k-step is
    int is = 0;
    TileRange itr = tile_at(walk[0]);
    uint32_t offa[4], offb[2];
    auto set_offsets = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            offa[i] = AKM ? (uint32_t)y * A.ld + itr.m0 + 64 * i + 8 * uu
                          : (itr.m0 + 64 * i + (uint32_t)y) * A.ld + 8 * uu;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            offb[i] = BKM ? (uint32_t)y * B.ld + itr.n0 + 64 * i + 8 * uu
                          : (itr.n0 + 64 * i + (uint32_t)y) * B.ld + 8 * uu;
    };
    set_offsets();
    constexpr uint32_t PAST = 0x80000000u;  // byte offset past every operand's range (< 2^31 bytes)
    // Loads of one k-step in two halves (A tiles 0-2, then A tile 3 and both B tiles), then the
    // cursor moves on.  The halves are issued after the products of each k-chunk: right after a
    // barrier all eight waves' loads reach the memory pipeline at once and a wave's issue stalls
    // until its loads are taken (hundreds of clocks for a step's 48 KB per CU); behind the
    // products that stall overlaps them.
    auto issue_half = [&](char *st, bool live, int half) {
        const uint32_t kk = itr.k0 + (uint32_t)is * CK;
        const uint32_t ka = AKM ? kk * A.ld : kk, kb = BKM ? kk * B.ld : kk;
        if (half == 0) {
#pragma unroll
            for (int i = 0; i < 3; ++i) lds_load16(A.rs, st + i * TBYTES + 1024 * w, live ? (offa[i] + ka) * 2 : PAST);
        } else {
            lds_load16(A.rs, st + 3 * TBYTES + 1024 * w, live ? (offa[3] + ka) * 2 : PAST);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                lds_load16(B.rs, st + (4 + i) * TBYTES + 1024 * w, live ? (offb[i] + kb) * 2 : PAST);
        }
    };
    auto advance_loads = [&](bool live) {
        if (live && ++is == itr.nk) {
            is = 0;
            if (++ij < walk.count) {
                itr = tile_at(walk[ij]);
                set_offsets();
            }
        }
    };
    auto issue_next = [&](char *st, bool live) {
        issue_half(st, live, 0);
        issue_half(st, live, 1);
        advance_loads(live);
    };

    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = zero4();
    uint32_t cj = 0;  // product cursor: tile cj, k-step cs of its cnk
    int cs = 0, cnk = itr.nk;
    // the products of one k-step from stage st, each k-chunk's followed by half of the loads of
    // the step after next into stage nxt (free: every wave is past its last read of it)
    auto compute = [&](const char *st, char *nxt, bool live) {
        const char *At = st + wm * TBYTES, *Bt = st + (4 + wn) * TBYTES;
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
            issue_half(nxt, live, kc);
        }
        advance_loads(live);
    };
    auto step = [&](char *cur, char *nxt, int g) {
        wait_vm_lgkm<6>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (cs == cnk - 2) pre(walk[cj]);
        compute(cur, nxt, g + 2 < S);
        if (++cs == cnk) {
            epi(walk[cj], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = zero4();
            cs = 0;
            if (++cj < walk.count) cnk = tile_at(walk[cj]).nk;
        }
    };
    issue_next(s0, true);
    issue_next(s1, S > 1);
    for (int g = 0;;) {
        step(s0, s2, g);
        if (++g == S) break;
        step(s1, s0, g);
        if (++g == S) break;
        step(s2, s1, g);
        if (++g == S) break;
    }
    wait_vm_lgkm<0>();  // the loads past the end
}

// max over the four lane groups (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float gmax(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

constexpr float LOG2E = 1.4426950408889634f;
__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * LOG2E); }
}  // namespace

// Forward tiles (class tile vt, token tile): A = W (rows = classes), B = h (rows = tokens), both
// k-contiguous.  part[vt][t] = (max, sum exp(logit - max)) over the tile's classes (the four waves
// of a token half combined through LDS), tl[t] = logit of token t's target (written by the one
// lane that holds it).
__global__ __launch_bounds__(CE_THREADS, 1) void la_ce_fwd_kernel(
    const bf16 *__restrict__ h, const bf16 *__restrict__ W, const int *__restrict__ targets,
    floatx2 *__restrict__ part, float *__restrict__ tl, int N, int d, int V, int Npad) {
    __shared__ __attribute__((aligned(16))) char s0[STAGE];
    __shared__ __attribute__((aligned(16))) char s1[STAGE];
    __shared__ __attribute__((aligned(16))) char s2[STAGE];
    __shared__ floatx2 xch[4 * NT];  // [4 wm][128 tokens]
    __shared__ int tg_lds[NT];       // the tile's targets, loaded before its epilogue
    // logical tile: the token tiles of one class tile consecutively (they share its rows of W)
    const uint32_t ntt = (uint32_t)Npad / NT, nvt = (uint32_t)(V + MT - 1) / MT;
    const Operand A{rsrc4(W, (uint32_t)V * d * 2), (uint32_t)d, false};
    const Operand B{rsrc4(h, (uint32_t)N * d * 2), (uint32_t)d, false};
    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w & 3, wn = w >> 2;
    const int4v trs = rsrc4(targets, (uint32_t)N * 4);
    auto tile_at = [&](uint32_t L) { return TileRange{(L / ntt) * MT, (L % ntt) * NT, 0u, d / CK}; };
    auto pre = [&](uint32_t L) {  // the two waves with wm = 0: 64 targets each
        if (wm == 0) lds_load4(trs, tg_lds + 64 * wn, ((L % ntt) * NT + 64 * wn + lane) * 4);
    };
    auto epi = [&](uint32_t L, floatx4 (&acc)[4][4]) {
        const uint32_t vt = L / ntt, v0 = vt * MT, t0 = (L % ntt) * NT;
        const int vbase = (int)v0 + 64 * wm + 4 * g;  // acc[i][j][e] is class vbase + 16 i + e
        const bool full = (int)v0 + MT <= V;          // no class of the tile past V (uniform)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int tloc = 64 * wn + 16 * j + r;
            const int t = (int)t0 + tloc;
            // the target's offset from the lane's first class: the lane holds its logit when it
            // is one of vbase + 16 i + e (rare: a branch, not a compare per element)
            const int q = tg_lds[tloc] - vbase;
            if ((unsigned)q < 64u && (q & 12) == 0 && t < N) {
                float x = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) x = q == 16 * i + e ? acc[i][j][e] : x;
                tl[t] = x;
            }
            float mx = -INFINITY, sum = 0.f;
            if (full) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, acc[i][j][e]);
                mx = gmax(mx);
                const float ml = -mx * LOG2E;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sum += __builtin_amdgcn_exp2f(fmaf(acc[i][j][e], LOG2E, ml));
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (vbase + 16 * i + e < V) mx = fmaxf(mx, acc[i][j][e]);
                mx = gmax(mx);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sum += vbase + 16 * i + e < V ? exp_f(acc[i][j][e] - mx) : 0.f;
            }
            sum = gsum(sum);
            if (g == 0) xch[wm * NT + tloc] = floatx2{mx, sum};
        }
        lds_barrier();
        if (tid < NT) {
            // a wave's classes may all lie past V (then max -inf, sum 0); the first wave's never do,
            // as no tile has V <= v0
            floatx2 x[4];
            float m = -INFINITY;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[k] = xch[k * NT + tid];
                m = fmaxf(m, x[k][0]);
            }
            float sm = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) sm += x[k][1] * exp_f(x[k][0] - m);
            part[(size_t)vt * Npad + t0 + tid] = floatx2{m, sm};
        }
        lds_barrier();  // xch is rewritten by the next tile's epilogue
    };
    gemm_tiles<false, false>(s0, s1, s2, A, B, TileWalk(nvt * ntt), tile_at, epi, pre);
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
__global__ __launch_bounds__(CE_THREADS, 1) void la_ce_p_kernel(
    const bf16 *__restrict__ h, const bf16 *__restrict__ W, const int *__restrict__ targets,
    const float *__restrict__ lse, const float *__restrict__ dloss, bf16 *__restrict__ P, int c0, int Nc, int N,
    int d, int V, int Vpad) {
    __shared__ __attribute__((aligned(16))) char s0[STAGE];
    __shared__ __attribute__((aligned(16))) char s1[STAGE];
    __shared__ __attribute__((aligned(16))) char s2[STAGE];
    __shared__ int tg_lds[NT];      // the tile's targets and lse, loaded before its epilogue
    __shared__ float lse_lds[NT];
    const uint32_t ntt = (uint32_t)(Nc + NT - 1) / NT, nvt = (uint32_t)Vpad / MT;
    const Operand A{rsrc4(W, (uint32_t)V * d * 2), (uint32_t)d, false};
    const Operand B{rsrc4(h + (size_t)c0 * d, (uint32_t)Nc * d * 2), (uint32_t)d, false};
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), wm = w & 3, wn = w >> 2;
    const float scale = (dloss ? *dloss : 1.f) / (float)N;
    const int4v trs = rsrc4(targets + c0, (uint32_t)Nc * 4), lrs = rsrc4(lse + c0, (uint32_t)Nc * 4);
    auto tile_at = [&](uint32_t L) { return TileRange{(L / ntt) * MT, (L % ntt) * NT, 0u, d / CK}; };
    auto pre = [&](uint32_t L) {  // the two waves with wm = 0: 64 tokens each
        if (wm == 0) {
            const uint32_t off = ((L % ntt) * NT + 64 * wn + lane) * 4;
            lds_load4(trs, tg_lds + 64 * wn, off);
            lds_load4(lrs, lse_lds + 64 * wn, off);
        }
    };
    auto epi = [&](uint32_t L, floatx4 (&acc)[4][4]) {
        const uint32_t v0 = (L / ntt) * MT, t0 = (L % ntt) * NT;
        // every class and token of the tile in range (uniform): no masks
        const bool full = (int)v0 + MT <= V && (int)t0 + NT <= Nc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int tloc = (int)t0 + 64 * wn + 16 * j + r;  // token within the chunk
            const int tgt = tg_lds[64 * wn + 16 * j + r];
            const float l = lse_lds[64 * wn + 16 * j + r];
            const bool live = tloc < Nc;
            const float ll = -l * LOG2E;
            uint32_t pk[4][2];  // P of classes vb(i) .. vb(i) + 3 in bf16, two per dword
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int vb = (int)v0 + 64 * wm + 16 * i + 4 * g;
                floatx4 p;
                if (full) {
                    const int q = tgt - vb;  // the target is element q of these four when 0 <= q < 4
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        p[e] = fmaf(__builtin_amdgcn_exp2f(fmaf(acc[i][j][e], LOG2E, ll)), scale,
                                    q == e ? -scale : 0.f);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int vv = vb + e;
                        const float x = exp_f(acc[i][j][e] - l) - (vv == tgt ? 1.f : 0.f);
                        p[e] = (live && vv < V) ? x * scale : 0.f;
                    }
                }
                const bf16x4 b4 = pack4(p);
                pk[i][0] = __builtin_bit_cast(uint2v, b4)[0];
                pk[i][1] = __builtin_bit_cast(uint2v, b4)[1];
            }
            // 16-byte stores: lanes of lane groups g and g ^ 1 trade pieces (the odd group's piece
            // of tile i for the even group's piece of tile i + 1), after which lane group g holds
            // eight consecutive classes, 16 (g & 1) + 8 (g >> 1) past the pair's first: each store
            // writes 64 contiguous bytes of 16 token rows
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                uint32_t lo[2], hi[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const auto sw = __builtin_amdgcn_permlane16_swap(pk[i][c], pk[i + 1][c], false, false);
                    lo[c] = sw[0];
                    hi[c] = sw[1];
                }
                const int vb = (int)v0 + 64 * wm + 16 * i + 16 * (g & 1) + 8 * (g >> 1);
                *reinterpret_cast<uint4v *>(P + (size_t)tloc * Vpad + vb) = uint4v{lo[0], lo[1], hi[0], hi[1]};
            }
        }
    };
    gemm_tiles<false, false>(s0, s1, s2, A, B, TileWalk(nvt * ntt), tile_at, epi, pre);
}

// dW tiles: C[m = feature][n = class] = sum_t h[t][m] P[t][n] over the chunk's (padded) tokens;
// both operands k-major.  Stored as dW[n][m] (fp32), or added to it (accumulate).  Features past d
// (the last feature tile when d is an odd multiple of 128) are not stored.
__global__ __launch_bounds__(CE_THREADS, 1) void la_ce_dw_kernel(const bf16 *__restrict__ h,
                                                                 const bf16 *__restrict__ P, float *__restrict__ dW,
                                                                 int c0, int Nc, int Ncpad, int d, int V, int Vpad,
                                                                 int accumulate) {
    __shared__ __attribute__((aligned(16))) char s0[STAGE];
    __shared__ __attribute__((aligned(16))) char s1[STAGE];
    __shared__ __attribute__((aligned(16))) char s2[STAGE];
    // the feature tiles of one class tile consecutively (they share its columns of P)
    const uint32_t nft = (uint32_t)(d + MT - 1) / MT, nct = (uint32_t)Vpad / NT;
    const Operand A{rsrc4(h + (size_t)c0 * d, (uint32_t)Nc * d * 2), (uint32_t)d, true};
    const Operand B{rsrc4(P, (uint32_t)Ncpad * Vpad * 2), (uint32_t)Vpad, true};
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), wm = w & 3, wn = w >> 2;
    auto tile_at = [&](uint32_t L) { return TileRange{(L % nft) * MT, (L / nft) * NT, 0u, Ncpad / CK}; };
    auto epi = [&](uint32_t L, floatx4 (&acc)[4][4]) {
        const uint32_t f0 = (L % nft) * MT, v0 = (L / nft) * NT;
        // d is a multiple of 128: a wave's 64 features lie all inside or all past it
        if ((int)f0 + 64 * wm >= d) return;
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
    };
    gemm_tiles<true, true>(s0, s1, s2, A, B, TileWalk(nft * nct), tile_at, epi);
}

// dh partial tiles: C[m = feature][n = token] = sum_v W[v][m] P[t][v] over the classes [k0, k1) of
// split z; A = W k-major, B = P k-contiguous.  Stored to part[z][t][m] (fp32), features past d
// excepted.
__global__ __launch_bounds__(CE_THREADS, 1) void la_ce_dh_kernel(const bf16 *__restrict__ W,
                                                                 const bf16 *__restrict__ P, float *__restrict__ part,
                                                                 int Ncpad, int d, int V, int Vpad, int kper,
                                                                 int nsplit) {
    __shared__ __attribute__((aligned(16))) char s0[STAGE];
    __shared__ __attribute__((aligned(16))) char s1[STAGE];
    __shared__ __attribute__((aligned(16))) char s2[STAGE];
    // split slowest, then token tile, feature tile fastest: consecutive tiles share P's rows of the
    // split, and the tiles of one split share its rows of W
    const uint32_t nft = (uint32_t)(d + MT - 1) / MT, ntt = (uint32_t)Ncpad / NT;
    const Operand A{rsrc4(W, (uint32_t)V * d * 2), (uint32_t)d, true};
    const Operand B{rsrc4(P, (uint32_t)Ncpad * Vpad * 2), (uint32_t)Vpad, false};
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), wm = w & 3, wn = w >> 2;
    auto tile_at = [&](uint32_t L) {
        const uint32_t z = L / (nft * ntt), rest = L % (nft * ntt);
        const uint32_t k0 = z * (uint32_t)kper;
        const uint32_t k1 = k0 + (uint32_t)kper < (uint32_t)Vpad ? k0 + (uint32_t)kper : (uint32_t)Vpad;
        return TileRange{(rest % nft) * MT, (rest / nft) * NT, k0, (int)((k1 - k0) / CK)};
    };
    auto epi = [&](uint32_t L, floatx4 (&acc)[4][4]) {
        const uint32_t z = L / (nft * ntt), rest = L % (nft * ntt);
        const uint32_t f0 = (rest % nft) * MT, t0 = (rest / nft) * NT;
        if ((int)f0 + 64 * wm >= d) return;
        float *base = part + (size_t)z * Ncpad * d;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = (int)t0 + 64 * wn + 16 * j + r;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<floatx4 *>(base + (size_t)t * d + f0 + 64 * wm + 16 * i + 4 * g) = acc[i][j];
        }
    };
    gemm_tiles<true, false>(s0, s1, s2, A, B, TileWalk(nft * ntt * (uint32_t)nsplit), tile_at, epi);
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

// Workgroups of a persistent launch over T tiles: one per compute unit at most (the GEMM kernels'
// LDS allows one), a multiple of 8 so that workgroup b runs on XCD b % 8 for every b; fewer when
// there are fewer tiles.
static unsigned persistent_grid(uint32_t T) {
    // CU count per device, read once (threads that race on the first read store the same value)
    static std::atomic<int> ncu[16];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
    int n = ncu[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) n = 8;
        ncu[dev].store(n, std::memory_order_relaxed);
    }
    const unsigned g = (unsigned)n / 8 * 8, t8 = (T + 7) / 8 * 8;
    return t8 < g ? t8 : g;
}

hipError_t launch_ce_fwd(const void *h, const void *W, const int *targets, float *loss, float *lse, void *ws, int N,
                         int d, int V, hipStream_t stream, const hipEvent_t ev[2]) {
    const CeShape s = ce_shape(N, d, V, N);
    floatx2 *part = reinterpret_cast<floatx2 *>(ws);
    float *tl = reinterpret_cast<float *>(static_cast<char *>(ws) + (size_t)s.nvt * s.Npad * 8);
    float *nll = tl + s.Npad;
    hipExtLaunchKernelGGL(la_ce_fwd_kernel, dim3(persistent_grid(s.nvt * (s.Npad / NT))), dim3(CE_THREADS), 0,
                          stream, ev[0], nullptr, 0, (const bf16 *)h, (const bf16 *)W, targets, part, tl, N, d, V,
                          s.Npad);
    hipExtLaunchKernelGGL(la_ce_lse_kernel, dim3((N + 15) / 16), dim3(256), 0, stream, nullptr, nullptr, 0,
                          (const floatx2 *)part, (const float *)tl, lse, nll, N, s.Npad, s.nvt);
    hipExtLaunchKernelGGL(la_ce_mean_kernel, dim3(1), dim3(1024), 0, stream, nullptr, ev[1], 0, (const float *)nll,
                          loss, N);
    return hipGetLastError();
}

// The forward's workspace for callers that cannot allocate one: one copy of this array per
// device the library runs on, held until the process ends, shared by every such call on that
// device (calls that overlap on one device race on it).  Its name in host code is a host-side
// stand-in, not a device address: the host uses only the address hipGetSymbolAddress gives for
// the current device, looked up once per device and kept.  The forward overwrites every byte of
// the workspace it reads, so nothing needs clearing between calls.
static __device__ __align__(256) char scratch[CE_SCRATCH_BYTES];
constexpr int SCRATCH_MAX_DEVICES = 64;
static std::atomic<void *> scratch_ptr[SCRATCH_MAX_DEVICES];

hipError_t launch_ce_fwd_noalloc(const void *h, const void *W, const int *targets, float *loss, float *lse, int N,
                                 int d, int V, hipStream_t stream, const hipEvent_t ev[2]) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
    void *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {  // first call on this device (threads that race here store the same address)
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return launch_ce_fwd(h, W, targets, loss, lse, p, N, d, V, stream, ev);
}

hipError_t launch_ce_bwd(const void *h, const void *W, const int *targets, const float *lse, const float *dloss,
                         void *dh, float *dW, void *ws, int N, int d, int V, int ce_chunk, hipStream_t stream,
                         const hipEvent_t ev[2]) {
    const CeShape s = ce_shape(N, d, V, ce_chunk);
    bf16 *P = static_cast<bf16 *>(ws);
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + s.p_bytes);
    for (int c0 = 0; c0 < N; c0 += s.chunk) {
        const int Nc = N - c0 < s.chunk ? N - c0 : s.chunk;
        const int Ncpad = (Nc + NT - 1) / NT * NT;
        const int nft = (d + MT - 1) / MT;
        const bool first = c0 == 0, last = c0 + s.chunk >= N;
        hipExtLaunchKernelGGL(la_ce_p_kernel, dim3(persistent_grid(s.nvt * (Ncpad / NT))), dim3(CE_THREADS), 0, stream,
                              first ? ev[0] : nullptr, nullptr, 0, (const bf16 *)h, (const bf16 *)W, targets, lse,
                              dloss, P, c0, Nc, N, d, V, s.Vpad);
        hipExtLaunchKernelGGL(la_ce_dh_kernel, dim3(persistent_grid(nft * (Ncpad / NT) * s.nsplit)), dim3(CE_THREADS),
                              0, stream, nullptr, nullptr, 0, (const bf16 *)W, (const bf16 *)P, part, Ncpad, d, V,
                              s.Vpad, s.kper, s.nsplit);
        const size_t n4 = (size_t)Nc * d / 4;
        hipExtLaunchKernelGGL(la_ce_dh_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                              nullptr, nullptr, 0, (const float *)part, (bf16 *)dh, c0, Nc, Ncpad, d, s.nsplit);
        hipExtLaunchKernelGGL(la_ce_dw_kernel, dim3(persistent_grid(nft * (s.Vpad / NT))), dim3(CE_THREADS), 0, stream, nullptr,
                              last ? ev[1] : nullptr, 0, (const bf16 *)h, (const bf16 *)P, dW, c0, Nc, Ncpad, d, V,
                              s.Vpad, first ? 0 : 1);
    }
    return hipGetLastError();
}

}  // namespace lachunk
