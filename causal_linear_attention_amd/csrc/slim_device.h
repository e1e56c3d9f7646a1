// slim_device.h -- device building blocks of the gfx950 kernels: operand
// fragments for the 16x16 MFMA shapes, tile staging through LDS, and the
// feature map g evaluated straight into MFMA register layouts.
//
// Fragment convention.  Every 16x16 fp32 accumulator block ("C block") held
// by a wave gives lane i the four entries (row 4*(i/16)+j, col i%16), j=0..3.
// An operand fragment Frag<T> carries, for one lane, four consecutive
// contraction indices 4*(i/16)..4*(i/16)+3 of one 16-wide contraction block,
// for the free index i%16.  Hence
//   * a C block Z (rows r, cols c) converts in registers into the operand of
//     any product that contracts over Z's rows, with Z's columns as the free
//     index (as the A operand of Z^T U or the B operand of U Z);
//   * an LDS array stored [n][k] (k contiguous) yields the operand for
//     contraction index k and free index n with one 8- or 16-byte read.
// Two 16-deep bf16 contraction blocks make one v_mfma_f32_16x16x32_bf16 (a lone
// block is zero-padded to 32); one fp32 block is four v_mfma_f32_16x16x4_f32
// (one per j).  A and B always pair the same physical indices, so
// the order in which an instruction walks its K dimension does not matter.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace slim {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

enum { FEAT_FAVOR = 0, FEAT_ELU1 = 1 };

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ int lcol() { return threadIdx.x & 15; }        // i % 16
__device__ __forceinline__ int lgrp() { return (threadIdx.x >> 4) & 3; }  // i / 16 (within the wave)

template <typename T> struct Frag;
template <> struct Frag<float> { f4 v; };
template <> struct Frag<__bf16> { bf4 v; };

__device__ __forceinline__ f4 f4zero() { return f4{0.f, 0.f, 0.f, 0.f}; }

template <typename T> __device__ __forceinline__ Frag<T> cfrag(f4 c);
template <> __device__ __forceinline__ Frag<float> cfrag<float>(f4 c) { return Frag<float>{c}; }
template <> __device__ __forceinline__ Frag<__bf16> cfrag<__bf16>(f4 c)
{
    Frag<__bf16> r;
    r.v[0] = (__bf16)c[0];
    r.v[1] = (__bf16)c[1];
    r.v[2] = (__bf16)c[2];
    r.v[3] = (__bf16)c[3];
    return r;
}

template <typename T> __device__ __forceinline__ f4 frag_to_f4(Frag<T> a);
template <> __device__ __forceinline__ f4 frag_to_f4<float>(Frag<float> a) { return a.v; }
template <> __device__ __forceinline__ f4 frag_to_f4<__bf16>(Frag<__bf16> a)
{
    return f4{(float)a.v[0], (float)a.v[1], (float)a.v[2], (float)a.v[3]};
}

// acc += A(16 x 16) * B(16 x 16) over one contraction block.
__device__ __forceinline__ void mma1(f4 &acc, Frag<float> a, Frag<float> b)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[0], b.v[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[1], b.v[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[2], b.v[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[3], b.v[3], acc, 0, 0, 0);
}
// bf16: a single 16-deep block also goes through v_mfma_f32_16x16x32_bf16, with the
// second half of both operands zero.  Every bf16 product therefore uses one MFMA
// kind: chaining v_mfma_f32_16x16x16_bf16 and v_mfma_f32_16x16x32_bf16 on the same
// accumulator was compiled without the wait states the hand-off needs on gfx950
// and produced wrong sums.
__device__ __forceinline__ void mma1(f4 &acc, Frag<__bf16> a, Frag<__bf16> b)
{
    const __bf16 z = (__bf16)0.f;
    bf8 a8 = {a.v[0], a.v[1], a.v[2], a.v[3], z, z, z, z};
    bf8 b8 = {b.v[0], b.v[1], b.v[2], b.v[3], z, z, z, z};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, acc, 0, 0, 0);
}
// acc += over two contraction blocks.
__device__ __forceinline__ void mma2(f4 &acc, Frag<float> a0, Frag<float> a1, Frag<float> b0, Frag<float> b1)
{
    mma1(acc, a0, b0);
    mma1(acc, a1, b1);
}
__device__ __forceinline__ void mma2(f4 &acc, Frag<__bf16> a0, Frag<__bf16> a1, Frag<__bf16> b0,
                                     Frag<__bf16> b1)
{
    bf8 a = {a0.v[0], a0.v[1], a0.v[2], a0.v[3], a1.v[0], a1.v[1], a1.v[2], a1.v[3]};
    bf8 b = {b0.v[0], b0.v[1], b0.v[2], b0.v[3], b1.v[0], b1.v[1], b1.v[2], b1.v[3]};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// acc += sum over contraction blocks kb = k0..k1-1 of A(kb) * B(kb); fa/fb return Frag<T>.
template <typename T, typename FA, typename FB>
__device__ __forceinline__ void mma_range(f4 &acc, int k0, int k1, FA fa, FB fb)
{
    int kb = k0;
    for (; kb + 1 < k1; kb += 2) mma2(acc, fa(kb), fa(kb + 1), fb(kb), fb(kb + 1));
    if (kb < k1) mma1(acc, fa(kb), fb(kb));
}

// The same over two contraction lists (blocks k0..k1-1 of fa/fb, then j0..j1-1 of
// ga/gb) into one accumulator, paired across the lists: an odd block of the first
// pairs with the second's first instead of going through a zero-padded product.
template <typename T, typename FA, typename FB, typename GA, typename GB>
__device__ __forceinline__ void mma_range2(f4 &acc, int k0, int k1, FA fa, FB fb, int j0, int j1, GA ga, GB gb)
{
    int kb = k0, jb = j0;
    for (; kb + 1 < k1; kb += 2) mma2(acc, fa(kb), fa(kb + 1), fb(kb), fb(kb + 1));
    if (kb < k1) {
        if (jb < j1) {
            mma2(acc, fa(kb), ga(jb), fb(kb), gb(jb));
            ++jb;
        } else {
            mma1(acc, fa(kb), fb(kb));
        }
    }
    for (; jb + 1 < j1; jb += 2) mma2(acc, ga(jb), ga(jb + 1), gb(jb), gb(jb + 1));
    if (jb < j1) mma1(acc, ga(jb), gb(jb));
}
// A-operand fragment of a 16-row block whose row 0 is all ones (the others zero):
// the product with it sums the B operand's contraction index into output row 0.
template <typename T> __device__ __forceinline__ Frag<T> ones_row0()
{
    const float o = lcol() == 0 ? 1.f : 0.f;
    return cfrag<T>(f4{o, o, o, o});
}

// Operand fragment from an LDS array stored [n][k] with row stride ld elements:
// free index n0 + i%16, contraction indices k0 + 4*(i/16) .. +3.
template <typename T> __device__ __forceinline__ Frag<T> lds_frag(const T *base, int ld, int n0, int k0)
{
    const T *p = base + (n0 + lcol()) * ld + k0 + 4 * lgrp();
    return *reinterpret_cast<const Frag<T> *>(p);
}

// Sum over the four lane groups (lanes i, i^16, i^32, i^48) of the same column.
__device__ __forceinline__ float sum_groups(float v)
{
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}
__device__ __forceinline__ float max_groups(float v)
{
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    v = fmaxf(v, __shfl_xor(v, 32, 64));
    return v;
}

__device__ __forceinline__ float fast_exp(float x)
{
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : fast_exp(x); }
__device__ __forceinline__ float elu1_grad(float x) { return x > 0.f ? 1.f : fast_exp(x); }

// 16-byte vector of the I/O type.
template <typename T> struct Vec16;
template <> struct Vec16<float> { typedef f4 type; static constexpr int N = 4; };
template <> struct Vec16<__bf16> { typedef bf8 type; static constexpr int N = 8; };

template <typename T> __device__ __forceinline__ typename Vec16<T>::type zero16()
{
    typename Vec16<T>::type z;
#pragma unroll
    for (int j = 0; j < Vec16<T>::N; ++j) z[j] = (T)0.f;
    return z;
}

// 16-byte vector store into an LDS row whose stride is only 8-byte aligned.
__device__ __forceinline__ void store16(float *p, f4 x) { *reinterpret_cast<f4 *>(p) = x; }
__device__ __forceinline__ void store16(__bf16 *p, bf8 x)
{
    reinterpret_cast<bf4 *>(p)[0] = bf4{x[0], x[1], x[2], x[3]};
    reinterpret_cast<bf4 *>(p)[1] = bf4{x[4], x[5], x[6], x[7]};
}

// Matrix in LDS, ROWS x COLS of the operand type T (COLS a multiple of 16).
// Operand fragments can contract over either index:
//   frag_c(n0, k0): free index = row n0 + i%16, contraction = columns k0 + 4g..+3;
//   frag_r(n0, k0): free index = column n0 + i%16, contraction = rows k0 + 4g..+3.
// bf16: column-blocked -- each 16-column block is its own ROWS x 16 array (32-byte
// rows), and within a row the 8-byte chunk q (0..3) is stored at q ^ ((r>>2)&3).
// Both read patterns (16 lanes over 16 rows of one chunk; 16 lanes over 4 rows x
// 4 chunks) then touch every bank once, and the address of a block at row or
// column offset n0, k0 (multiples of 16) is a fixed offset from the lane's base
// address, so one address register serves every block.  frag_r is one
// ds_read_b64_tr_b16 (within each 16-lane group, lane i receives element i%4 of
// the chunks addressed by lanes i/4, 4+i/4, 8+i/4, 12+i/4, so lane L points at
// row k0+4g+L/4, column n0+4(L%4)).  fp32: row-major with rows padded by 4
// elements, frag_r is four 4-byte reads.  PAD (bf16) spaces the column blocks by
// PAD extra elements: a matrix written row-wise across blocks (the staged input
// tiles: each thread stores 8 consecutive columns) would otherwise put the same
// row of different blocks on the same banks.
template <typename T, int ROWS, int COLS, int PAD = 0> struct LMat {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr int LD = BF ? COLS : COLS + 4;
    static constexpr int BSTRIDE = ROWS * 16 + PAD;  // bf16: elements per 16-column block
    static constexpr int SIZE = BF ? (COLS / 16) * BSTRIDE : ROWS * LD;
    static_assert(COLS % 16 == 0, "columns: a multiple of 16");
    T *p;
    __device__ __forceinline__ explicit LMat(T *base) : p(base) {}
    __device__ static __forceinline__ int off(int r, int c)  // c % 4 == 0
    {
        if constexpr (BF)
            return (c >> 4) * BSTRIDE + r * 16 + ((((c >> 2) & 3) ^ ((r >> 2) & 3)) << 2);
        else
            return r * LD + c;
    }
    // four consecutive columns c..c+3 of row r
    __device__ __forceinline__ void put4(int r, int c, f4 v) const
    {
        if constexpr (BF)
            *reinterpret_cast<bf4 *>(p + off(r, c)) = bf4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        else
            *reinterpret_cast<f4 *>(p + off(r, c)) = v;
    }
    __device__ __forceinline__ void put_frag(int r, int c, Frag<T> v) const
    {
        *reinterpret_cast<Frag<T> *>(p + off(r, c)) = v;
    }
    // one 16-byte vector of the I/O type at columns c..c+EPV-1 (c % EPV == 0)
    __device__ __forceinline__ void put16(int r, int c, typename Vec16<T>::type x) const
    {
        if constexpr (BF) {
            *reinterpret_cast<bf4 *>(p + off(r, c)) = bf4{x[0], x[1], x[2], x[3]};
            *reinterpret_cast<bf4 *>(p + off(r, c + 4)) = bf4{x[4], x[5], x[6], x[7]};
        } else {
            *reinterpret_cast<f4 *>(p + off(r, c)) = x;
        }
    }
    __device__ __forceinline__ f4 get4(int r, int c) const
    {
        if constexpr (BF) {
            const bf4 v = *reinterpret_cast<const bf4 *>(p + off(r, c));
            return f4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
        } else {
            return *reinterpret_cast<const f4 *>(p + off(r, c));
        }
    }
    __device__ __forceinline__ Frag<T> frag_c(int n0, int k0) const
    {
        return *reinterpret_cast<const Frag<T> *>(p + off(n0 + lcol(), k0 + 4 * lgrp()));
    }
    __device__ __forceinline__ Frag<T> frag_r(int n0, int k0) const
    {
        if constexpr (BF) {
            const int L = lcol();
            const T *a = p + off(k0 + 4 * lgrp() + (L >> 2), n0 + 4 * (L & 3));
            typedef __attribute__((address_space(3))) bf4 lds_bf4;
            Frag<T> f;
            f.v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf4 *)(a));
            return f;
        } else {
            Frag<T> f;
            const int r = k0 + 4 * lgrp(), c = n0 + lcol();
#pragma unroll
            for (int j = 0; j < 4; ++j) f.v[j] = p[(r + j) * LD + c];
            return f;
        }
    }
};

// Orders this wave's LDS writes before its later LDS reads of the same
// locations (per-wave scratch in LDS, no other wave involved).
__device__ __forceinline__ void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Floats per row of the backward's row statistics: 1/den, dden, the query
// feature offset (exp2 domain) and one unused.
constexpr int ROWSTAT = 4;
// Rows per workgroup of the row-statistics kernel (its grid splits each chunk in parts).
constexpr int ROWSTAT_ROWS = 256;

// Key-side offset of the FAVOR+ map, one number per projection W.  For every key
// k and feature m, w_m.k - |k|^2/2 = |w_m|^2/2 - |k - w_m|^2/2 <= |w_m|^2/2, so
// with koff = max(0, max_m |w_m|^2/2 - KOFF_MARGIN) every key feature evaluated
// as exp(w_m.k - |k|^2/2 - koff)/sqrt(M) is at most exp(KOFF_MARGIN)/sqrt(M),
// whatever the keys: fp32 cannot overflow, and the prefix sums of up to 2^31 rows
// of such features times values of moderate size stay finite.  A factor common to
// all key features cancels in Y and in every input gradient (eq. (2) is
// homogeneous of degree 0 in the keys' features taken together), so only the
// states that cross the boundary carry it.  For the usual draws (|w_m|^2 near d,
// d <= 64) koff is 0 and nothing changes.
constexpr float KOFF_MARGIN = 60.f;

// koff of W [M][D] (fp32, or bf16 when wbf16), computed by a whole workgroup of
// at least M threads (every thread must call it; it synchronises the workgroup).
// Thread m sums its row's squares in index order; the maximum over rows is exact in
// any order, so every kernel that calls this gets the same value bit for bit.
// red: LDS scratch of one float per wave of the workgroup, plus one.
__device__ __forceinline__ float key_offset_block(const void *W, int wbf16, int M, int D, float *red)
{
    float n2 = 0.f;
    if ((int)threadIdx.x < M) {
        // row m's squares summed in index order; its elements fetched 16 bytes at a time
        // (rows start 16-byte aligned: W is, and D is a multiple of 16)
        if (wbf16) {
            const uint4 *row = reinterpret_cast<const uint4 *>((const uint16_t *)W + (size_t)threadIdx.x * D);
#pragma unroll 4
            for (int j = 0; j < D / 8; ++j) {
                const uint4 u = row[j];
                const unsigned p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float lo = __uint_as_float(p[h] << 16), hi = __uint_as_float(p[h] & 0xffff0000u);
                    n2 = fmaf(lo, lo, n2);
                    n2 = fmaf(hi, hi, n2);
                }
            }
        } else {
            const float4 *row = reinterpret_cast<const float4 *>((const float *)W + (size_t)threadIdx.x * D);
#pragma unroll 4
            for (int j = 0; j < D / 4; ++j) {
                const float4 u = row[j];
                n2 = fmaf(u.x, u.x, n2);
                n2 = fmaf(u.y, u.y, n2);
                n2 = fmaf(u.z, u.z, n2);
                n2 = fmaf(u.w, u.w, n2);
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) n2 = fmaxf(n2, __shfl_xor(n2, o, 64));
    const int nw = (blockDim.x + 63) / 64;
    if (lane_id() == 0) red[wave_id()] = n2;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = red[0];
        for (int w = 1; w < nw; ++w) m = fmaxf(m, red[w]);
        red[nw] = fmaxf(0.f, 0.5f * m - KOFF_MARGIN);
    }
    __syncthreads();
    return red[nw];
}

// A [TT][D] tile of a row-major tensor held in registers: thread i owns the
// 16-byte vectors i, i+NT, ... (row t = idx / VPR, columns c..c+EPV-1).  load()
// issues the global reads (rows >= nvalid read as zero) and returns at once, so a
// tile can be fetched while the previous one is being computed; store() moves it
// into LDS once the data is needed.
// The same pointer, moved to scalar registers (it must be uniform across the wave).
// Tile loads then address base + 32-bit lane offset, so the compiler keeps one small
// offset per lane instead of a 64-bit pointer per tensor and lane across the tile loop.
template <typename T> __device__ __forceinline__ const T *uniform_ptr(const T *p)
{
    const unsigned long long a = (unsigned long long)p;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
    return (const T *)(((unsigned long long)hi << 32) | lo);
}
// Load through a global-memory pointer (a pointer rebuilt from integers is generic,
// which would make the compiler emit flat loads), marked non-temporal: the tiles are
// read once, and streaming them keeps the caches for what is reused (W, W^T).
template <typename U> __device__ __forceinline__ U gload(const void *p)
{
    return __builtin_nontemporal_load((const __attribute__((address_space(1))) U *)p);
}

template <typename T, int D, int TT, int NT> struct TileRegs {
    typedef typename Vec16<T>::type V;
    static constexpr int EPV = Vec16<T>::N;
    static constexpr int VPR = D / EPV;
    static constexpr int NV = TT * VPR;
    static constexpr int PER = (NV + NT - 1) / NT;
    V v[PER];
    float s[PER];

    // stats (optional): per-row records of sstride floats whose first is the row's
    // scale; row t's scale goes with its vectors.
    __device__ __forceinline__ void load(const T *__restrict__ src, int nvalid, const float *stats = nullptr,
                                         int sstride = ROWSTAT)
    {
        const T *base = uniform_ptr(src);
        const float *sbase = stats ? uniform_ptr(stats) : nullptr;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + i * NT;
            const int t = idx / VPR, c = (idx % VPR) * EPV;
            const bool ok = idx < NV && t < nvalid;
            v[i] = ok ? gload<V>(base + (unsigned)(t * D + c)) : zero16<T>();
            if (stats) s[i] = ok ? gload<float>(sbase + (unsigned)(t * sstride)) : 0.f;
        }
    }
    // Move the tile into an LDS matrix (rows t, columns e); scaled: multiply row t
    // by its stats scale first; rowfn (if not null) is called by one lane per
    // row as rowfn(t, |row t|^2) (summed over the VPR lanes of the row).
    template <class MAT, class RF>
    __device__ __forceinline__ void store(const MAT &dst, bool scaled, RF rowfn) const
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + i * NT;
            const int t = idx / VPR, c = (idx % VPR) * EPV;
            V x = v[i];
            if (scaled) {
#pragma unroll
                for (int j = 0; j < EPV; ++j) x[j] = (T)((float)x[j] * s[i]);
            }
            if (idx < NV) dst.put16(t, c, x);
            if constexpr (!std::is_same<RF, std::nullptr_t>::value) {
                float q = 0.f;
#pragma unroll
                for (int j = 0; j < EPV; ++j) q += (float)x[j] * (float)x[j];
#pragma unroll
                for (int o = 1; o < VPR; o <<= 1) q += __shfl_xor(q, o, 64);
                if (idx < NV && c == 0) rowfn(t, q);
            }
        }
    }
    // rows t >= nvalid of the tile hold `fill` instead of zero after load()
    __device__ __forceinline__ void fill_invalid(int nvalid, float fill)
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = threadIdx.x + i * NT;
            if (idx / VPR >= nvalid) {
#pragma unroll
                for (int j = 0; j < EPV; ++j) v[i][j] = (T)fill;
            }
        }
    }
};

// Per-row statistics of a tile held in registers by threads 0..TT-1.
template <int TT> struct RowStatRegs {
    float inv, dd, qoff;
    __device__ __forceinline__ void load(const float *st, int nvalid)
    {
        const int t = threadIdx.x;
        const bool ok = t < TT && t < nvalid;
        const float *sb = uniform_ptr(st) + (unsigned)(t * ROWSTAT);
        inv = ok ? gload<float>(sb) : 0.f;
        dd = ok ? gload<float>(sb + 1) : 0.f;
        qoff = ok ? gload<float>(sb + 2) : 0.f;
    }
};

}  // namespace slim
