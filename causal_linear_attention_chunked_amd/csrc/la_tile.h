// Building blocks of the 128-token kernels (two 64-token blocks, D = 64, bf16
// elements): swizzled 64 x 64 bf16 tiles in LDS, per-lane fragment offsets, a
// cheap hi + lo operand split and wave-level row reductions.
//
// Tile layout.  A tile is 64 rows of 64 bf16 (128 bytes, no padding).  Its
// 8-byte units (4 elements) are XOR-swizzled by row: unit u of row y sits at
// unit u ^ swz(y).  With that map the three access patterns the kernels use are
// all free of LDS bank conflicts (64 banks of 4 bytes):
//   - the natural fragment read (lane: row r, units g and g + 4 of a k-chunk),
//   - the transposed fragment read (ds_read_b64_tr_b16: lane (g, m, a) reads
//     row 4g + m, unit a of a 16-column slab),
//   - the 16-byte staging write (8 threads per row).
// swz() only uses the low four bits of the row and is even, so a fragment of 16
// rows starting at a multiple of 16 sees the same per-lane offsets in every row
// slab, and 16-byte pairs of units stay contiguous.
#pragma once
#include "la_common.h"

namespace lachunk {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

constexpr int TROW = 128;            // bytes per tile row
constexpr int TBYTES = 64 * TROW;    // bytes per tile

__device__ __forceinline__ int swz(int row) { return ((row ^ (row >> 1)) & 7) << 1; }

// Per-lane byte offsets inside a tile.
//   nat(u): natural fragment of rows 16*rt + (lane & 15), units 4u + g: the operand
//           fragment of k-chunk kc is units u = 2kc (slots 0-3) and 2kc + 1 (slots 4-7);
//           the same offsets address a bf16x4 accumulator write of output tile
//           (m-tile u, n-tile rt) stored as [n][m].
//   tr(u) : transposed fragment of the 16 storage columns 16u..16u+15 (the operand's rows),
//           storage rows 4g + m of a 16-row slab (add 16 * slab * TROW).
// nat[] / tr[] hold the four values for compile-time indices; nat_at() / tr_at() compute
// one for a run-time index (an array indexed at run time would live in scratch memory).
// `base` is added to every offset: tiles at 64 KB and above are addressed as (tile - base) +
// offset with base held opaquely in a register, so that the ds instructions' 16-bit offset
// field takes the rest (otherwise every access pays an add).
struct TileLanes {
    int rrow, ln, trow, lt, g, sr;
    uint32_t base;
    uint32_t nat[4], tr[4];
    __device__ __forceinline__ explicit TileLanes(int lane, uint32_t base_ = 0) {
        const int r = lane & 15, g = lane >> 4, m = (lane & 15) >> 2, a = lane & 3;
        base = base_;
        rrow = r * TROW;
        this->g = g;
        sr = swz(r);
        ln = g ^ swz(r);
        trow = (4 * g + m) * TROW;
        lt = a ^ swz(4 * g + m);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            nat[u] = nat_at(u);
            tr[u] = tr_at(u);
        }
    }
    __device__ __forceinline__ uint32_t nat_at(int u) const { return base + rrow + 8 * ((4 * u) ^ ln); }
    __device__ __forceinline__ uint32_t tr_at(int u) const { return base + trow + 8 * ((4 * u) ^ lt); }
};

// A uniform value in a register the compiler cannot see through (for TileLanes::base).
__device__ __forceinline__ uint32_t opaque_v(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Volatile, so that the two 8-byte halves of different fragments are never merged into one
// ds_read2 (which would land them in the wrong registers and cost a v_mov per dword).
typedef __attribute__((address_space(3))) const volatile bf16x4 lds_vbf16x4;
__device__ __forceinline__ bf16x4 lds_b64(const char *p) { return *(lds_vbf16x4 *)(p); }

// Operand fragment of tile rows 16*rt..+15 (row, k contiguous), k-chunk kc.
__device__ __forceinline__ bf16x8 tfrag(const char *tile, const TileLanes &L, int rt, int kc) {
    const char *b = tile + rt * 16 * TROW;
    return __builtin_shufflevector(lds_b64(b + L.nat[2 * kc]), lds_b64(b + L.nat[2 * kc + 1]), 0, 1, 2, 3, 4, 5, 6, 7);
}
// The same for a k-chunk known only at run time.
__device__ __forceinline__ bf16x8 tfrag_at(const char *tile, const TileLanes &L, int rt, int kc) {
    const char *b = tile + rt * 16 * TROW;
    return __builtin_shufflevector(lds_b64(b + L.nat_at(2 * kc)), lds_b64(b + L.nat_at(2 * kc + 1)), 0, 1, 2, 3, 4, 5,
                                   6, 7);
}
// Operand fragment of tile rows 16*rt..+15 in the contiguous k order: lane (r, g) holds
// elements 32kc + 8g..+7 of its row (one 16-byte read).  Both operands of a product must
// use the same k order; this one pairs with cfrag_g() and crowfrag().
__device__ __forceinline__ bf16x8 tfrag_c(const char *tile, const TileLanes &L, int rt, int kc) {
    return *reinterpret_cast<const bf16x8 *>(tile + rt * 16 * TROW + L.rrow + 8 * ((8 * kc + 2 * (L.g)) ^ L.sr));
}
// Operand fragment of the transpose: operand rows are storage columns 16u..+15 where
// troff = TileLanes::tr(u), k = storage rows 32*kc..+31.
__device__ __forceinline__ bf16x8 tfrag_tr(const char *tile, uint32_t troff, int kc) {
    const char *b = tile + kc * 32 * TROW + troff;
    const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(b));
    const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(b + 16 * TROW));
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4, 5,
                                   6, 7);
}
// Writes an accumulator tile (lane: n = lane & 15, m = 4g + i) as bf16 into storage row
// 16*nt + n, columns 16*mt + 4g..+3, where natoff = TileLanes::nat(mt).
__device__ __forceinline__ void tstore_acc(char *tile, uint32_t natoff, int nt, const bf16x4 &x) {
    *reinterpret_cast<bf16x4 *>(tile + nt * 16 * TROW + natoff) = x;
}
// Writes an operand fragment (rows 16*rt + lane&15, k-chunk kc) into a tile stored
// "row, k contiguous": the inverse of tfrag().
__device__ __forceinline__ void tstore_frag(char *tile, const TileLanes &L, int rt, int kc, const bf16x8 &f) {
    char *b = tile + rt * 16 * TROW;
    *reinterpret_cast<bf16x4 *>(b + L.nat[2 * kc]) = __builtin_shufflevector(f, f, 0, 1, 2, 3);
    *reinterpret_cast<bf16x4 *>(b + L.nat[2 * kc + 1]) = __builtin_shufflevector(f, f, 4, 5, 6, 7);
}
// The same for a k-chunk known only at run time.
__device__ __forceinline__ void tstore_frag_at(char *tile, const TileLanes &L, int rt, int kc, const bf16x8 &f) {
    char *b = tile + rt * 16 * TROW;
    *reinterpret_cast<bf16x4 *>(b + L.nat_at(2 * kc)) = __builtin_shufflevector(f, f, 0, 1, 2, 3);
    *reinterpret_cast<bf16x4 *>(b + L.nat_at(2 * kc + 1)) = __builtin_shufflevector(f, f, 4, 5, 6, 7);
}
// Byte offset of a thread's 16-byte staging slot (8 threads per 128-byte row).
__device__ __forceinline__ uint32_t stage_off(int tid) {
    const int row = tid >> 3, c = tid & 7;
    return row * TROW + 8 * ((2 * c) ^ swz(row));
}

// Workgroup barrier that orders LDS only.  __syncthreads() fences every address space, so
// each wave would first wait for its own outstanding global loads and stores; here the
// waves exchange data through LDS alone, and outputs stored to global memory before a
// barrier keep draining across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders a wave's LDS writes before its later LDS reads of what other lanes of the same wave
// wrote.  A wave's LDS operations complete in issue order, so no workgroup barrier is needed; the
// fences keep the compiler from moving the reads above the writes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Store of four bf16 outputs (8 bytes per lane; the four lanes of an accumulator row write
// 32 contiguous bytes per instruction).  Non-temporal (NT) or write-back.  A one-chunk
// launch is faster with non-temporal stores, at the price of partial-sector writes (more
// HBM write bytes than the tensor size); a workgroup that walks many chunks is much faster
// with write-back stores, whose lines the L2 completes before they go out.
// LA_BF16_NT_STORES=0 makes every store write-back.
#ifndef LA_BF16_NT_STORES
#define LA_BF16_NT_STORES 1
#endif
template <bool NT>
__device__ __forceinline__ void store_bf16x4(bf16 *p, const bf16x4 &x) {
    if (NT && LA_BF16_NT_STORES) __builtin_nontemporal_store(x, reinterpret_cast<bf16x4 *>(p));
    else *reinterpret_cast<bf16x4 *>(p) = x;
}

// Positive feature map phi(x) = elu(x) + 1 (alpha = 1): x + 1 above zero, e^x below; eight bf16
// inputs mapped in fp32 (e^x as 2^(x log2 e) on the transcendental unit) and rounded to bf16.
// Since e^x >= x + 1 everywhere, phi(x) = max(x + 1, min(e^x, 1)): the min is the exp's output
// clamp to [0, 1], and no compare and select is needed.
__device__ __forceinline__ float elu1_f(float f) {
    const float e = __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(f * 1.4426950408889634f), 0.f, 1.f);
    return __builtin_fmaxf(f + 1.f, e);
}
__device__ __forceinline__ bf16x8 elu1_8(const bf16x8 &x) {
    bf16x8 y;
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = (bf16)elu1_f((float)x[i]);
    return y;
}
// phi'(x) from the mapped value: 1 above zero (where phi > 1), e^x = phi below.
__device__ __forceinline__ floatx4 elu1_grad4(const bf16x4 &phi) {
    floatx4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_fminf((float)phi[i], 1.f);
    return r;
}

// a -= p exactly as the unevaluated sum a + c: the rounding error of the fp32 difference
// (Knuth's two-sum on a and -p) is added to the compensation term c.
__device__ __forceinline__ void two_diff(float &a, float &c, float p) {
    const float x = a, y = -p;
    const float s = x + y;
    const float yy = s - x;
    const float err = (x - (s - yy)) + (y - yy);
    a = s;
    c += err;
}
__device__ __forceinline__ void two_sum(float &a, float &c, float p) { two_diff(a, c, -p); }
__device__ __forceinline__ void two_sum4(floatx4 &a, floatx4 &c, const floatx4 &p) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float ae = a[e], ce = c[e];
        two_diff(ae, ce, -p[e]);
        a[e] = ae;
        c[e] = ce;
    }
}
// The unevaluated sum a + c as its fp32 rounding s and the exact remainder res = (a + c) - s,
// for any magnitudes of a and c (Knuth's branch-free two-sum: a compensation term may outgrow
// a running sum whose terms cancel).  Host-callable, so that a CPU test can check it.
__host__ __device__ __forceinline__ void fold(float a, float c, float &s, float &res) {
    s = a + c;
    const float cc = s - a;
    res = (a - (s - cc)) + (c - cc);
}
__device__ __forceinline__ void two_diff4(floatx4 &a, floatx4 &c, const floatx4 &p) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float ae = a[e], ce = c[e];
        two_diff(ae, ce, p[e]);
        a[e] = ae;
        c[e] = ce;
    }
}

// bf16x4 of four fp32 values (round to nearest even)
__device__ __forceinline__ bf16x4 pack4(const floatx4 &x) {
    const bf16x2 a{(bf16)x[0], (bf16)x[1]}, b{(bf16)x[2], (bf16)x[3]};
    return __builtin_bit_cast(bf16x4, (uint32_t __attribute__((ext_vector_type(2)))){__builtin_bit_cast(uint32_t, a),
                                                                                       __builtin_bit_cast(uint32_t, b)});
}

// The selector pairs (-1, 0) and (0, -1) of split_pair, as scalar registers the compiler
// cannot fold into an instruction constant.  Folded, the pair (-1, 0) becomes the inline
// constant -1.0, which v_dot2c_f32_bf16 reads as the 32-bit pattern 0xBF800000, i.e.
// the pair (0, -1): the wrong element.
__device__ __forceinline__ bf16x2 opaque_pair(uint32_t bits) {
    asm("" : "+s"(bits));
    return __builtin_bit_cast(bf16x2, bits);
}

// hi = bf16(x), lo = bf16(x - hi): the difference is exact in fp32 and comes from one
// v_dot2_f32_bf16 per element (-hi * 1 + x), so a pair costs four VALU operations.
__device__ __forceinline__ void split_pair(float x0, float x1, bf16x2 &hi, bf16x2 &lo) {
    hi = bf16x2{(bf16)x0, (bf16)x1};
    const bf16x2 m0 = opaque_pair(0x0000BF80u), m1 = opaque_pair(0xBF800000u);
    const float d0 = __builtin_amdgcn_fdot2_f32_bf16(hi, m0, x0, false);
    const float d1 = __builtin_amdgcn_fdot2_f32_bf16(hi, m1, x1, false);
    lo = bf16x2{(bf16)d0, (bf16)d1};
}
struct Split8 {
    bf16x8 hi, lo;
};
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bits(const bf16x2 &x) { return __builtin_bit_cast(uint32_t, x); }
// Split of two accumulator tiles (k 0..15 from a0, 16..31 from a1) as one operand fragment;
// the packed pairs are placed whole (no per-element repacking).
__device__ __forceinline__ Split8 split_acc(const floatx4 &a0, const floatx4 &a1) {
    bf16x2 h[4], l[4];
    split_pair(a0[0], a0[1], h[0], l[0]);
    split_pair(a0[2], a0[3], h[1], l[1]);
    split_pair(a1[0], a1[1], h[2], l[2]);
    split_pair(a1[2], a1[3], h[3], l[3]);
    Split8 s;
    s.hi = __builtin_bit_cast(bf16x8, u32x4{bits(h[0]), bits(h[1]), bits(h[2]), bits(h[3])});
    s.lo = __builtin_bit_cast(bf16x8, u32x4{bits(l[0]), bits(l[1]), bits(l[2]), bits(l[3])});
    return s;
}
__device__ __forceinline__ void split4(const floatx4 &x, bf16x4 &hi, bf16x4 &lo) {
    bf16x2 h0, l0, h1, l1;
    split_pair(x[0], x[1], h0, l0);
    split_pair(x[2], x[3], h1, l1);
    hi = __builtin_bit_cast(bf16x4, u32x2{bits(h0), bits(h1)});
    lo = __builtin_bit_cast(bf16x4, u32x2{bits(l0), bits(l1)});
}

// acc += X Y^T with X split (hi + lo) and Y exact, or the other way round.
__device__ __forceinline__ void mma_s(floatx4 &acc, const Split8 &x, const bf16x8 &y) {
    mma(acc, x.hi, y);
    mma(acc, x.lo, y);
}
__device__ __forceinline__ void mma_s(floatx4 &acc, const bf16x8 &x, const Split8 &y) {
    mma(acc, x, y.hi);
    mma(acc, x, y.lo);
}

// Sum over the four lane groups (lanes l, l^16, l^32, l^48) with the gfx950 lane swaps.
__device__ __forceinline__ float gsum(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Operand fragment in the contiguous k order straight from global memory: rows of a
// "row, k contiguous" matrix (pitch ld elements), `base` = element offset of (row0, k0).
__device__ __forceinline__ bf16x8 cfrag_g(const GRes &gr, uint32_t base, int ld, int lane) {
    return gload<bf16x8>(gr, (base + (lane & 15) * ld + 8 * (lane >> 4)) * 2);
}
// A row vector (bf16, 64 entries, unswizzled) as an operand whose 16 rows are all that row,
// contiguous k order.
__device__ __forceinline__ bf16x8 crowfrag(const char *row, int lane, int kc) {
    return *reinterpret_cast<const bf16x8 *>(row + 2 * (32 * kc + 8 * (lane >> 4)));
}

// Operand fragment whose 16 rows are all the same row vector (bf16, 64 entries, unswizzled):
// slot s of lane (r, g) is element 32kc + kslot.
__device__ __forceinline__ bf16x8 rowfrag(const char *row, int lane, int kc) {
    const char *p = row + 2 * (32 * kc + 4 * (lane >> 4));
    return __builtin_shufflevector(lds_b64(p), lds_b64(p + 32), 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace lachunk
