// Device building blocks shared by the forward and backward kernels: element
// types, 16x16 MFMA tiles on gfx950, operand fragments and LDS staging.
//
// Tile convention.  Every product is C = X Y^T over a contraction index k, with
// X (rows m) and Y (rows n) both stored "row, k contiguous".  One 16x16 output
// tile lives in a floatx4 per lane: lane l, element i holds C[4*(l/16)+i][l%16].
// A k-chunk of 32 is one v_mfma_f32_16x16x32_bf16 (bf16) or eight
// v_mfma_f32_16x16x4_f32 (fp32).  Inside a chunk, lane-group g = l/16 and slot
// s = 0..7 carry k = 16*(s/4) + 4*g + (s%4), for X and Y alike.  With that map
// two adjacent output tiles (k 0..15 and 16..31 of the next product) are already
// a ready operand fragment: an accumulator becomes the next MFMA's operand with
// no data movement, its fixed lane index (n) being the operand's row and its
// per-lane index (m) the contraction index.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lachunk {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

constexpr int BK = 64;      // tokens per block of the blocked form
constexpr int NWAVE = 8;    // waves per workgroup: two per SIMD
constexpr int NTHR = 512;   // threads per workgroup

template <typename T> struct Elem;
template <> struct Elem<float> {
    using frag = floatx8;   // one k-chunk of 32: eight single-float operands
    using vec4 = floatx4;   // four consecutive elements (16 bytes)
    static constexpr int PAD = 4;   // LDS row padding, elements
};
template <> struct Elem<bf16> {
    using frag = bf16x8;    // one k-chunk of 32: one 8-element operand
    using vec4 = bf16x4;    // four consecutive elements (8 bytes)
    static constexpr int PAD = 8;
};

template <typename T> using Frag = typename Elem<T>::frag;
template <typename T> using Vec4 = typename Elem<T>::vec4;

__device__ __forceinline__ float tof(float x) { return x; }
__device__ __forceinline__ float tof(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T fromf(float x) { return (T)x; }

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// acc += X_chunk * Y_chunk^T over one k-chunk of 32.
__device__ __forceinline__ void mma(floatx4 &acc, const bf16x8 &a, const bf16x8 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(floatx4 &acc, const floatx8 &a, const floatx8 &b) {
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
}

// Operand fragment of 16 rows x one k-chunk from a "row, k contiguous" matrix.
// `base` points at (row0, k0); `ld` is the row pitch in elements (a multiple of 4).
template <typename T>
__device__ __forceinline__ Frag<T> ldfrag(const T *base, int ld, int lane) {
    const T *p = base + (lane & 15) * ld + 4 * (lane >> 4);
    Vec4<T> a = *reinterpret_cast<const Vec4<T> *>(p);
    Vec4<T> b = *reinterpret_cast<const Vec4<T> *>(p + 16);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Same, every element multiplied by a per-lane scale (rounded once to T).
template <typename T>
__device__ __forceinline__ Frag<T> ldfrag_scaled(const T *base, int ld, int lane, float scale) {
    const T *p = base + (lane & 15) * ld + 4 * (lane >> 4);
    Vec4<T> a = *reinterpret_cast<const Vec4<T> *>(p);
    Vec4<T> b = *reinterpret_cast<const Vec4<T> *>(p + 16);
    Frag<T> f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        f[s] = fromf<T>(tof(a[s]) * scale);
        f[s + 4] = fromf<T>(tof(b[s]) * scale);
    }
    return f;
}

// Operand fragment from two accumulator tiles covering k 0..15 (a0) and 16..31 (a1).
template <typename T>
__device__ __forceinline__ Frag<T> frag_acc(const floatx4 &a0, const floatx4 &a1) {
    Frag<T> f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        f[s] = fromf<T>(a0[s]);
        f[s + 4] = fromf<T>(a1[s]);
    }
    return f;
}

// k index (within its chunk) of slot s for this lane.
__device__ __forceinline__ int kslot(int lane, int s) { return 16 * (s >> 2) + 4 * (lane >> 4) + (s & 3); }

__device__ __forceinline__ Vec4<float> cvt4(const floatx4 &x, float) { return x; }
__device__ __forceinline__ Vec4<bf16> cvt4(const floatx4 &x, bf16) {
    return bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
}
template <typename T> __device__ __forceinline__ Vec4<T> to_vec4(const floatx4 &x) { return cvt4(x, T()); }

__device__ __forceinline__ float wsum_g(float x) {
    // sum over the four lane-groups (lanes l, l^16, l^32, l^48)
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// Transposed operand fragment: 16 rows x one k-chunk of X where X is stored
// "k, row contiguous" (X^T row-major, pitch ld).  `base` points at (k0, row0).
// bf16 uses the gfx950 LDS transpose read: in each 16-lane group the lanes
// supply 16 addresses of 4 consecutive elements, and lane i gets element i%4 of
// the rows supplied by lanes i/4, 4+i/4, 8+i/4, 12+i/4.  Addressing lane
// (m = (l%16)/4, a = l%4) of group g at stored row k0 + 4g + m, column row0 + 4a
// therefore hands lane (r = l%16, g) the four k values 4g..4g+3 of row r, which
// is slots 0..3 of the fragment; rows k0 + 16 + ... give slots 4..7.  fp32 reads
// the same elements one by one.
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

template <typename T>
__device__ __forceinline__ Frag<T> ldfrag_tr(const T *base, int ld, int lane) {
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
        const int g = lane >> 4, m = (lane & 15) >> 2, a = lane & 3;
        const T *p = base + (4 * g + m) * ld + 4 * a;
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(p));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(p + 16 * ld));
        f = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi),
                                    0, 1, 2, 3, 4, 5, 6, 7);
    } else {
        const T *p = base + (lane & 15);
#pragma unroll
        for (int s = 0; s < 8; ++s) f[s] = p[kslot(lane, s) * ld];
    }
    return f;
}

// ---------------------------------------------------------------------------
// Split operands.  An fp32 intermediate x (scores, gradients, the running
// state) enters a bf16 MFMA as hi + lo with hi = bf16(x), lo = bf16(x - hi):
// about 16 mantissa bits instead of 8.  Exact operands (the bf16 inputs) are
// used as they are, so a product of a split and an exact operand takes two
// MFMAs and a product of two split operands three (hi*hi + hi*lo + lo*hi).  With
// fp32 elements every fragment is exact and each product is one fp32 MFMA chain.
template <typename T> struct SFrag {
    Frag<T> hi, lo;
};

template <typename T> __device__ __forceinline__ constexpr bool is_bf16() { return sizeof(T) == 2; }

template <typename T>
__device__ __forceinline__ SFrag<T> split8(const floatx8 &x) {
    SFrag<T> f;
    if constexpr (is_bf16<T>()) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const bf16 h = (bf16)x[s];
            f.hi[s] = h;
            f.lo[s] = (bf16)(x[s] - (float)h);
        }
    } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) f.hi[s] = x[s];
    }
    return f;
}

template <typename T>
__device__ __forceinline__ void mma_sx(floatx4 &acc, const SFrag<T> &x, const Frag<T> &y) {
    mma(acc, x.hi, y);
    if constexpr (is_bf16<T>()) mma(acc, x.lo, y);
}
template <typename T>
__device__ __forceinline__ void mma_xs(floatx4 &acc, const Frag<T> &x, const SFrag<T> &y) {
    mma(acc, x, y.hi);
    if constexpr (is_bf16<T>()) mma(acc, x, y.lo);
}
template <typename T>
__device__ __forceinline__ void mma_ss(floatx4 &acc, const SFrag<T> &x, const SFrag<T> &y) {
    mma(acc, x.hi, y.hi);
    if constexpr (is_bf16<T>()) {
        mma(acc, x.hi, y.lo);
        mma(acc, x.lo, y.hi);
    }
}

// fp32 fragment values from two accumulator tiles (k 0..15 and 16..31), times `scale`
__device__ __forceinline__ floatx8 acc8(const floatx4 &a0, const floatx4 &a1, float scale = 1.f) {
    return floatx8{a0[0] * scale, a0[1] * scale, a0[2] * scale, a0[3] * scale,
                   a1[0] * scale, a1[1] * scale, a1[2] * scale, a1[3] * scale};
}
// fp32 fragment values from an fp32 LDS matrix stored "row, k contiguous"
__device__ __forceinline__ floatx8 ld8_rows(const float *base, int ld, int lane) {
    const float *p = base + (lane & 15) * ld + 4 * (lane >> 4);
    const floatx4 a = *reinterpret_cast<const floatx4 *>(p);
    const floatx4 b = *reinterpret_cast<const floatx4 *>(p + 16);
    return floatx8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// fp32 fragment values from an fp32 LDS matrix stored "k, row contiguous" (the transpose):
// base points at (k0, row0); element (k, row) at base[k * ld + row]
__device__ __forceinline__ floatx8 ld8_cols(const float *base, int ld, int lane) {
    floatx8 f;
    const float *p = base + (lane & 15);
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = p[kslot(lane, s) * ld];
    return f;
}
// fp32 values of an element-type fragment, each slot multiplied by sc[s]
template <typename T>
__device__ __forceinline__ floatx8 ld8_scaled(const T *base, int ld, int lane, const floatx8 &sc) {
    const Frag<T> f = ldfrag<T>(base, ld, lane);
    floatx8 x;
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] = tof(f[s]) * sc[s];
    return x;
}
template <typename T>
__device__ __forceinline__ floatx8 ld8_scaled(const T *base, int ld, int lane, float sc) {
    const Frag<T> f = ldfrag<T>(base, ld, lane);
    floatx8 x;
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] = tof(f[s]) * sc;
    return x;
}
// Split fragment read from stored hi / lo copies (lo is not read for fp32 elements).
template <typename T>
__device__ __forceinline__ SFrag<T> ldsplit(const T *hi, const T *lo, int ld, int lane) {
    SFrag<T> f;
    f.hi = ldfrag<T>(hi, ld, lane);
    if constexpr (is_bf16<T>()) f.lo = ldfrag<T>(lo, ld, lane);
    return f;
}
template <typename T>
__device__ __forceinline__ SFrag<T> ldsplit_tr(const T *hi, const T *lo, int ld, int lane) {
    SFrag<T> f;
    f.hi = ldfrag_tr<T>(hi, ld, lane);
    if constexpr (is_bf16<T>()) f.lo = ldfrag_tr<T>(lo, ld, lane);
    return f;
}
// fp32 values of an element fragment
template <typename T> __device__ __forceinline__ floatx8 tof8(const Frag<T> &f) {
    floatx8 x;
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] = tof(f[s]);
    return x;
}
// Writes four consecutive fp32 values as hi (and lo for bf16) element copies.
template <typename T>
__device__ __forceinline__ void store_split4(T *hi, T *lo, const floatx4 &x) {
    if constexpr (is_bf16<T>()) {
        bf16x4 h, l;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h[i] = (bf16)x[i];
            l[i] = (bf16)(x[i] - (float)h[i]);
        }
        *reinterpret_cast<bf16x4 *>(hi) = h;
        *reinterpret_cast<bf16x4 *>(lo) = l;
    } else {
        *reinterpret_cast<floatx4 *>(hi) = x;
    }
}

template <typename T> __device__ __forceinline__ Frag<T> ones_frag() {
    Frag<T> f;
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = fromf<T>(1.f);
    return f;
}

// ---------------------------------------------------------------------------
// Global reads go through buffer resources: a base address and a byte range.
// A read past the range returns zero without touching memory, so ragged rows,
// blocks past the end of a chunk and an absent (NULL) carry need no branches,
// and every load of a prefetch can be issued unconditionally.  Offsets are byte
// offsets from the base (32-bit: the host keeps each per-group range below 2 GiB).
// Keeps every load issued above this point above it: neither the IR optimiser
// (a memory clobber) nor the machine scheduler may move memory operations across.
// Used right after a prefetch is issued, so the loads go out early.
__device__ __forceinline__ void issue_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

struct GRes {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ GRes(const void *base, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000)) {}
};
template <typename V> __device__ __forceinline__ V gload(const GRes &g, uint32_t off) {
    static_assert(sizeof(V) == 4 || sizeof(V) == 8 || sizeof(V) == 16, "buffer load width");
    if constexpr (sizeof(V) == 16) {
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(g.r, off, 0, 0));
    } else if constexpr (sizeof(V) == 8) {
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(g.r, off, 0, 0));
    } else {
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b32(g.r, off, 0, 0));
    }
}
// Operand fragment straight from global memory ("row, k contiguous", pitch ld elements);
// `base` is the element offset of (row0, k0).
template <typename T>
__device__ __forceinline__ Frag<T> ldfrag_g(const GRes &g, uint32_t base, int ld, int lane) {
    const uint32_t e = base + (lane & 15) * ld + 4 * (lane >> 4);
    const Vec4<T> a = gload<Vec4<T>>(g, e * sizeof(T));
    const Vec4<T> b = gload<Vec4<T>>(g, (e + 16) * sizeof(T));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------
// LDS staging of a [64][NCOL] tile read from global memory (row pitch `gld`
// elements) through registers: load() issues the 16-byte reads, store() writes
// LDS later, so a block's loads are in flight while the previous block computes.
//   nat : if non-null, [rows][ldn] natural copy
//   tr  : if non-null, [NCOL][ldt] transposed copy (tr[c][row])
template <typename T, int NCOL>
struct Stager {
    static constexpr int VE = 16 / sizeof(T);         // elements per 16-byte vector
    static constexpr int VPR = NCOL / VE;              // vectors per row
    static constexpr int NV = BK * VPR;                // vectors per 64-row tile
    static constexpr int PER = (NV + NTHR - 1) / NTHR; // vectors per thread
    typedef T vec_t __attribute__((ext_vector_type(16 / sizeof(T))));

    vec_t r[PER];

    static_assert(NV % NTHR == 0, "every thread stages whole vectors");
    // rows past the resource's range (past the chunk) read as zero
    __device__ __forceinline__ void load(const GRes &g, uint32_t base, int gld, int tid) {
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const int vi = tid + it * NTHR;
            const int row = vi / VPR, cv = vi % VPR;
            r[it] = gload<vec_t>(g, (base + (uint32_t)(row * gld + cv * VE)) * sizeof(T));
        }
    }
    // row `row` times 1/den[row], written as hi (and lo for bf16) element copies
    __device__ __forceinline__ void store_scaled_split(T *hi, T *lo, int ldn, const float *den, int tid) const {
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            int vi = tid + it * NTHR;
            int row = vi / VPR, cv = vi % VPR;
            if (vi < NV) {
                const float s = 1.f / den[row];
                vec_t h, l;
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const float x = tof(r[it][e]) * s;
                    h[e] = fromf<T>(x);
                    l[e] = fromf<T>(x - tof(h[e]));
                }
                *reinterpret_cast<vec_t *>(hi + row * ldn + cv * VE) = h;
                if (sizeof(T) == 2) *reinterpret_cast<vec_t *>(lo + row * ldn + cv * VE) = l;
            }
        }
    }
    __device__ __forceinline__ void store(T *nat, int ldn, T *tr, int ldt, int tid) const {
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            int vi = tid + it * NTHR;
            int row = vi / VPR, cv = vi % VPR;
            if (vi < NV) {
                if (nat) *reinterpret_cast<vec_t *>(nat + row * ldn + cv * VE) = r[it];
                if (tr) {
#pragma unroll
                    for (int e = 0; e < VE; ++e) tr[(cv * VE + e) * ldt + row] = r[it][e];
                }
            }
        }
    }
};

}  // namespace lachunk
