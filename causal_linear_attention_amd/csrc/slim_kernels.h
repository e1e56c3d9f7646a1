// slim_kernels.h -- the gfx950 kernels of the chunked causal linear attention.
//
// Method (page "Sub-Linear Memory: How to Make Performers SLiM"):
//   Subsection 2.1, eq. (2)-(4): Y_l = R_l g(Q_l) / (S_l . g(Q_l)) with the prefix
//     sums R_l = sum_{i<=l} V_i g(K_i)^T (d x M) and S_l = sum_{i<=l} g(K_i) (M);
//   Subsection 3.2, eq. (14)-(18): the sequence is cut into N slices ("chunks") of
//     length c, the last one possibly shorter, and each slice's prefix sums start
//     from the previous slice's final state;
//   Subsection 3.3, updates (19)-(20): the backward walks the slices in reverse,
//     recovering each slice's entry state from the final one by subtracting the
//     slice's own contribution, and carrying the gradient of the state, which is a
//     prefix sum taken backwards.
//
// GPU decomposition.  One workgroup owns one (head, chunk).  Inside a chunk it
// walks tiles of TT rows (the page's "block" form of the iterative prefix sum,
// Section 4), carrying the d x M state in registers.  The NW waves of a
// workgroup split the M features: wave w owns features [w*MW, (w+1)*MW), holds
// its slice of every feature-indexed matrix (g(Q), g(K), R, S and their
// gradients) in MFMA accumulator layout, and reduces the feature-contracted
// outputs (numerators, dQ, dK, dV) across waves through LDS.  Waves are kept to
// 4 per workgroup where the state fits (64 features per wave), and a kernel whose
// LDS fits twice in a compute unit is compiled for 2 waves per SIMD, so two
// workgroups share each compute unit and hide each other's barrier waits.
//
// Augmented value index.  V, the state R, dNum and dR carry one extra 16-wide
// block of the value index e whose first column is 1 (V), S (R), dden (dNum) or
// dS (dR), the rest zero.  With it the MFMAs produce, as that extra column, the
// denominators (sum_s P[t][s] + g(Q_t).S), S += sum g(K), the dden.S and dS terms
// of the gradients and the rank-one part of A = dNum V^T + dden 1^T.
//
// Every LDS tile is stored row-major only; fragments that contract over its rows
// use gfx950's transposing LDS read (LMat::frag_r).
//
// Kernels (all launched on a grid (chunks in window, B*H)):
//   featmap_kernel : standalone g(X), optional per-row max offset.
//   state_kernel   : dR_n = sum_{rows of chunk n} V g(K)^T, dS_n = sum g(K).
//   scan_kernel    : per-head sequential sweep over the window's chunk states with
//                    an fp64 carry (forward prefix, window start by subtraction,
//                    gradient suffix sum, plain accumulation).
//   fwd_kernel     : Y for a chunk from its entry state.
//   stats_kernel   : backward pass 1: recompute the chunk forward, emit per-row
//                    1/den and dden = -(dY.Y)/den.
//   bwdq_kernel    : dQ (forward tile order, entry state R), and the chunk's
//                    gradient contribution to its entry state,
//                    dG_n = sum dNum g(Q)^T (and dden g(Q)).
//   bwdkv_kernel   : dK, dV (reverse tile order, gradient state dR).
#pragma once
#include "slim_device.h"

namespace slim {

struct ChunkArgs {
    const void *Q, *K, *V, *W, *dY;
    const void *Wt;            // W^T fragments, packed (backward, FAVOR+)
    void *out0, *out1, *out2;  // fwd: Y | bwdq: dQ | bwdkv: dK, dV
    float *slots;              // [BH][P+1][(D+1)*M]  state slots (R rows, then S)
    float *gslots;             // [BH][P+1][(D+1)*M]  gradient-state slots
    float *stats;              // [BH][P][c][ROWSTAT] per-row (1/den, dden, query offset, -)
    void *pq, *pk;             // dW pass: dg(Q).g(Q), dg(K).g(K) [BH][P][c][M] (operand type)
    float *rstat;              // [BH][L][2] per row (1/den, query offset): written by the forward,
                               // read by the backward instead of recomputing them (or NULL)
    const void *Yin;           // backward with the forward's row statistics: its output Y
    const float *koff;         // FAVOR+: the key-side offset of W (key_offset_block), one float
    long long L;
    int c;   // chunk length
    int n0;  // first chunk of the window
    int P;   // window capacity (slot stride)
};

constexpr float LOG2E = 1.4426950408889634f;

// MW_ = features per wave (0: 64 for bf16 with d <= 64 when that still leaves 4
// waves, else 32 -- 64 keeps a wave's fp32 state blocks and fragments within 256
// registers only at d <= 64, and workgroups of fewer than 4 waves leave too little
// work in flight per compute unit: one-wave workgroups at M = 64 ran 2.2x slower).
// PADX_ = bf16 elements between the 16-column blocks of the staged input tiles (see LMat).
template <typename T_, int D_, int M_, int FEAT_, int TT_, int MW_ = 0, int PADX_ = 32> struct KCfg {
    typedef T_ T;
    static constexpr int D = D_, M = M_, FEAT = FEAT_, TT = TT_;
    static constexpr int MWA = MW_ ? MW_ : ((sizeof(T_) == 2 && D_ <= 64 && M_ >= 256) ? 64 : 32);
    static constexpr int MW = M >= MWA ? MWA : M;  // features per wave
    static constexpr int NW = M / MW;              // waves per workgroup
    static constexpr int NT = NW * 64;
    static constexpr int NFB = MW / 16;
    static constexpr int NEB = D / 16;
    static constexpr int NEA = NEB + 1;  // value blocks including the auxiliary one
    static constexpr int NTB = TT / 16;
    static constexpr int LDR = D + 4;  // fp32 reduction rows; column D = denominator / row sum
    static constexpr int SZ = (D + 1) * M;
    static constexpr bool FAVOR = FEAT == FEAT_FAVOR;
    typedef TileRegs<T, D, TT, NT> Tile;
    typedef LMat<T, TT, D, PADX_> XMat;  // [TT][D] input tile
    typedef LMat<T, TT, 16> AuxMat;  // auxiliary value block of a tile (column 0 used)
    typedef LMat<T, TT, MW> FMat;    // one wave's features of a tile: rows t, columns m
    static_assert(FEAT == FEAT_FAVOR || D == M, "elu+1 needs M == d");
    static_assert(MW % 16 == 0 && D % 16 == 0 && TT % 16 == 0, "block sizes");
};

// Waves per SIMD a kernel is compiled for (its register budget): 2 when two of
// its workgroups fit a compute unit's 160 KB of LDS and 4 SIMDs, so that one
// workgroup's barriers and memory waits overlap the other's work; else 1.
constexpr int waves_per_simd(size_t lds_bytes, int nw) { return (nw <= 4 && 2 * lds_bytes <= 160 * 1024) ? 2 : 1; }

// A value-indexed tile (V or dNum) with its auxiliary block.
template <class C> struct AugTile {
    typedef typename C::T T;
    typename C::XMat x;
    typename C::AuxMat a;
    __device__ __forceinline__ AugTile(T *main, T *aux) : x(main), a(aux) {}
    // free index row n0 + i%16, contraction over value block eb
    __device__ __forceinline__ Frag<T> fc(int n0, int eb) const
    {
        return eb < C::NEB ? x.frag_c(n0, eb * 16) : a.frag_c(n0, 0);
    }
    // free index value block eb, contraction over rows k0 + 4g..
    __device__ __forceinline__ Frag<T> fr(int eb, int k0) const
    {
        return eb < C::NEB ? x.frag_r(eb * 16, k0) : a.frag_r(0, k0);
    }
    // row t of the auxiliary block: (v, 0, ..., 0); one lane per row.
    __device__ __forceinline__ void set_aux(int t, float v) const
    {
        a.put4(t, 0, f4{v, 0.f, 0.f, 0.f});
        a.put4(t, 4, f4zero());
        a.put4(t, 8, f4zero());
        a.put4(t, 12, f4zero());
    }
};

// ------------------------------------------------------------------ g(X) ---

// W fragments of this wave's features: wf[fb][kb] holds W[m][kb*16 + 4g..+3] for
// m = w*MW + fb*16 + i%16 (free index m, contraction over d).
template <class C>
__device__ __forceinline__ void load_wfrag(Frag<typename C::T> (&wf)[C::NFB][C::NEB], const void *Wv)
{
    typedef typename C::T T;
    const T *W = (const T *)Wv;
    const int w = wave_id();
#pragma unroll
    for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
        for (int kb = 0; kb < C::NEB; ++kb)
            wf[fb][kb] = *reinterpret_cast<const Frag<T> *>(
                W + (size_t)(w * C::MW + fb * 16 + lcol()) * C::D + kb * 16 + 4 * lgrp());
}

// W^T fragments: wt[eb][fb] holds W[m][e] for m = w*MW + fb*16 + 4g + j, e = eb*16 + i%16
// (free index e, contraction over this wave's features).  Block eb = NEB (if
// present) is the auxiliary column of ones (e = D), which turns the product into
// the row sum over m.
template <class C, int NE>
__device__ __forceinline__ void load_wtfrag(Frag<typename C::T> (&wt)[NE][C::NFB], const void *Wv)
{
    typedef typename C::T T;
    const T *W = (const T *)Wv;
    const int w = wave_id();
#pragma unroll
    for (int eb = 0; eb < NE; ++eb)
#pragma unroll
        for (int fb = 0; fb < C::NFB; ++fb) {
            Frag<T> f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                f.v[j] = eb < C::NEB ? W[(size_t)(w * C::MW + fb * 16 + 4 * lgrp() + j) * C::D + eb * 16 + lcol()]
                                     : (T)(lcol() == 0 ? 1.f : 0.f);
            wt[eb][fb] = f;
        }
}

// One value block eb (< NEB) of the W^T fragments above, from the fragment-packed
// copy Wp of W: for feature block mb (16 features) and value block eb, the 64
// lanes' fragments lie in one contiguous 512-byte run, lane i holding
// W[mb*16 + 4(i/16) + j][eb*16 + i%16], j = 0..3.
template <class C>
__device__ __forceinline__ void load_wtfrag_block(Frag<typename C::T> (&wt)[C::NFB], const void *Wpv, int eb)
{
    typedef typename C::T T;
    const T *Wp = (const T *)Wpv;
    const int mb0 = wave_id() * (C::MW / 16);
#pragma unroll
    for (int fb = 0; fb < C::NFB; ++fb)
        wt[fb] = *reinterpret_cast<const Frag<T> *>(Wp + (((size_t)eb * (C::M / 16) + mb0 + fb) * 64 + threadIdx.x % 64) * 4);
}

// Feature blocks in "transposed" orientation: ph[fb][tb] has rows m = w*MW + fb*16 + 4g + j
// and columns t = tb*16 + i%16.  FAVOR+: the raw projection w_m . x_t.  elu+1: g itself.
template <class C>
__device__ __forceinline__ void feat_T(f4 (&ph)[C::NFB][C::NTB], const typename C::XMat &xs,
                                       const Frag<typename C::T> (&wf)[C::NFB][C::NEB])
{
    typedef typename C::T T;
#pragma unroll
    for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
        for (int tb = 0; tb < C::NTB; ++tb) {
            if constexpr (C::FAVOR) {
                f4 acc = f4zero();
                mma_range<T>(acc, 0, C::NEB, [&](int kb) { return wf[fb][kb]; },
                             [&](int kb) { return xs.frag_c(tb * 16, kb * 16); });
                ph[fb][tb] = acc;
            } else {
                f4 x = frag_to_f4<T>(xs.frag_c(tb * 16, wave_id() * C::MW + fb * 16));
                ph[fb][tb] = f4{elu1(x[0]), elu1(x[1]), elu1(x[2]), elu1(x[3])};
            }
        }
}

// Feature blocks in "token" orientation: ph[tb][fb] has rows t = tb*16 + 4g + j and
// columns m = w*MW + fb*16 + i%16 (elu+1 reads the tile transposed).
template <class C>
__device__ __forceinline__ void feat_S(f4 (&ph)[C::NTB][C::NFB], const typename C::XMat &xs,
                                       const Frag<typename C::T> (&wf)[C::NFB][C::NEB])
{
    typedef typename C::T T;
#pragma unroll
    for (int tb = 0; tb < C::NTB; ++tb)
#pragma unroll
        for (int fb = 0; fb < C::NFB; ++fb) {
            if constexpr (C::FAVOR) {
                f4 acc = f4zero();
                mma_range<T>(acc, 0, C::NEB, [&](int kb) { return xs.frag_c(tb * 16, kb * 16); },
                             [&](int kb) { return wf[fb][kb]; });
                ph[tb][fb] = acc;
            } else {
                f4 x = frag_to_f4<T>(xs.frag_r(wave_id() * C::MW + fb * 16, tb * 16));
                ph[tb][fb] = f4{elu1(x[0]), elu1(x[1]), elu1(x[2]), elu1(x[3])};
            }
        }
}

// FAVOR+ query offsets: this wave's maximum of w_m . q_t over its features, per t.
template <class C> __device__ __forceinline__ void q_partial_max(const f4 (&ph)[C::NFB][C::NTB], float *qmax)
{
#pragma unroll
    for (int tb = 0; tb < C::NTB; ++tb) {
        float m = -3.0e38f;
#pragma unroll
        for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
            for (int j = 0; j < 4; ++j) m = fmaxf(m, ph[fb][tb][j]);
        m = max_groups(m);
        if (lgrp() == 0) qmax[wave_id() * C::TT + tb * 16 + lcol()] = m;
    }
}

// g(K) exactly: exp(w_m.k_t - |k_t|^2/2) / sqrt(M) = 2^(log2e w_m.k_t - kn2[t]) with
// kn2[t] = log2e (|k_t|^2/2 + ln(M)/2), +inf for rows beyond the chunk (g = 0 there).
// elu+1 rows beyond the chunk were staged as -inf, so g = 0 there too.
// g(Q) is evaluated up to a positive per-row factor, which cancels in Y and in dQ
// (Y is homogeneous of degree 0 in each g(Q_l)).
// Queries with this wave's own row maximum as offset: g'(Q_t) = g(Q_t) * exp(-m_w(t))
// with m_w(t) = max over the wave's features of w_m . q_t, recorded in qmax[w][t] for
// the cross-wave sums, which rescale each wave's partials to the common maximum
// (no barrier is needed here).  elu+1: nothing to do.
template <class C> __device__ __forceinline__ void q_wave_finish(f4 (&ph)[C::NFB][C::NTB], float *qmax)
{
    if constexpr (C::FAVOR) {
#pragma unroll
        for (int tb = 0; tb < C::NTB; ++tb) {
            float m = -3.0e38f;
#pragma unroll
            for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
                for (int j = 0; j < 4; ++j) m = fmaxf(m, ph[fb][tb][j]);
            m = max_groups(m);
            if (lgrp() == 0) qmax[wave_id() * C::TT + tb * 16 + lcol()] = m;
            const float off = -m * LOG2E;
#pragma unroll
            for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
                for (int j = 0; j < 4; ++j) ph[fb][tb][j] = __builtin_amdgcn_exp2f(fmaf(ph[fb][tb][j], LOG2E, off));
        }
    }
}
// Per-wave scale factors of tile row t: sc[w] = exp(m_w(t) - max_w' m_w'(t)) (all 1 for
// elu+1); *moff = the common offset -max * log2 e (0 for elu+1).
template <class C> __device__ __forceinline__ void wave_scales(const float *qmax, int t, float (&sc)[C::NW], float *moff)
{
    if constexpr (C::FAVOR) {
        float m = qmax[t];
#pragma unroll
        for (int w = 1; w < C::NW; ++w) m = fmaxf(m, qmax[w * C::TT + t]);
#pragma unroll
        for (int w = 0; w < C::NW; ++w) sc[w] = __builtin_amdgcn_exp2f((qmax[w * C::TT + t] - m) * LOG2E);
        *moff = -m * LOG2E;
    } else {
#pragma unroll
        for (int w = 0; w < C::NW; ++w) sc[w] = 1.f;
        *moff = 0.f;
    }
}

// Queries with a known per-row offset (exp2 domain, -rowmax * log2 e): qoff[t] for
// tile row t (the backward reads it from the row statistics the
// stats pass wrote, so it needs no cross-wave maximum).  elu+1: nothing to do.
template <class C> __device__ __forceinline__ void q_finish_off(f4 (&ph)[C::NFB][C::NTB], const float *qoff)
{
    if constexpr (C::FAVOR) {
#pragma unroll
        for (int tb = 0; tb < C::NTB; ++tb) {
            const float off = qoff[tb * 16 + lcol()];
#pragma unroll
            for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
                for (int j = 0; j < 4; ++j) ph[fb][tb][j] = __builtin_amdgcn_exp2f(fmaf(ph[fb][tb][j], LOG2E, off));
        }
    }
}
template <class C> __device__ __forceinline__ void k_finish_T(f4 (&ph)[C::NFB][C::NTB], const float *kn2)
{
    if constexpr (C::FAVOR) {
#pragma unroll
        for (int tb = 0; tb < C::NTB; ++tb) {
            const float off = -kn2[tb * 16 + lcol()];
#pragma unroll
            for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
                for (int j = 0; j < 4; ++j) ph[fb][tb][j] = __builtin_amdgcn_exp2f(fmaf(ph[fb][tb][j], LOG2E, off));
        }
    }
}
template <class C> __device__ __forceinline__ void k_finish_S(f4 (&ph)[C::NTB][C::NFB], const float *kn2)
{
    if constexpr (C::FAVOR) {
#pragma unroll
        for (int tb = 0; tb < C::NTB; ++tb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float off = -kn2[tb * 16 + 4 * lgrp() + j];
#pragma unroll
                for (int fb = 0; fb < C::NFB; ++fb)
                    ph[tb][fb][j] = __builtin_amdgcn_exp2f(fmaf(ph[tb][fb][j], LOG2E, off));
            }
    }
}

// Row function for staging K: kn2[t] as above, plus the key-side offset koff of W
// (every key feature scaled by exp(-koff); see key_offset_block).
template <class C> struct KnormFn {
    float *kn2;
    int nv;
    float koff;
    __device__ __forceinline__ void operator()(int t, float q) const
    {
        kn2[t] = t < nv ? (0.5f * q + 0.5f * __logf((float)C::M) + koff) * LOG2E : __builtin_inff();
    }
};

// The key-side offset of the call (0 for elu+1), a uniform scalar load.
template <class C> __device__ __forceinline__ float key_off(const ChunkArgs &a)
{
    if constexpr (C::FAVOR)
        return *a.koff;
    else
        return 0.f;
}

// Write this wave's feature blocks ph[fb][tb] (rows m, cols t) into F (rows t, cols m).
template <class C>
__device__ __forceinline__ void put_features(const typename C::FMat &F, const f4 (&ph)[C::NFB][C::NTB])
{
#pragma unroll
    for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
        for (int tb = 0; tb < C::NTB; ++tb) F.put4(tb * 16 + lcol(), fb * 16 + 4 * lgrp(), ph[fb][tb]);
}

// Same, from the blocks already converted to operand fragments (no second conversion).
template <class C>
__device__ __forceinline__ void put_feature_frags(const typename C::FMat &F,
                                                  const Frag<typename C::T> (&f)[C::NFB][C::NTB])
{
#pragma unroll
    for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
        for (int tb = 0; tb < C::NTB; ++tb) F.put_frag(tb * 16 + lcol(), fb * 16 + 4 * lgrp(), f[fb][tb]);
}

template <class C, int A, int B>
__device__ __forceinline__ void to_frags(Frag<typename C::T> (&f)[A][B], const f4 (&c)[A][B])
{
#pragma unroll
    for (int a = 0; a < A; ++a)
#pragma unroll
        for (int b = 0; b < B; ++b) f[a][b] = cfrag<typename C::T>(c[a][b]);
}

// Sum the NW per-wave fp32 partials red[w][t][e] for tile rows and hand
// (t, e..e+3, value, row valid) to `emit`.
template <class C, typename F>
__device__ __forceinline__ void reduce_rows(const float *red, int nv, F emit)
{
    constexpr int Q4 = C::D / 4;
    for (int v = threadIdx.x; v < C::TT * Q4; v += C::NT) {
        const int t = v / Q4, e = (v % Q4) * 4;
        f4 s = *reinterpret_cast<const f4 *>(red + t * C::LDR + e);
#pragma unroll
        for (int w = 1; w < C::NW; ++w) s += *reinterpret_cast<const f4 *>(red + (w * C::TT + t) * C::LDR + e);
        emit(t, e, s, t < nv);
    }
}
// Sum over waves of column D of the reduction rows (denominator / row sum) of row t.
template <class C> __device__ __forceinline__ float reduce_col(const float *red, int t)
{
    float s = red[t * C::LDR + C::D];
#pragma unroll
    for (int w = 1; w < C::NW; ++w) s += red[(w * C::TT + t) * C::LDR + C::D];
    return s;
}
// Write a value-indexed block acc (rows e = eb*16 + 4g + j, cols t = tb*16 + i%16) of
// this wave's partial to red; the auxiliary block contributes only column D.
template <class C> __device__ __forceinline__ void put_red(float *red, int eb, int tb, f4 acc)
{
    const int row = (wave_id() * C::TT + tb * 16 + lcol()) * C::LDR;
    if (eb < C::NEB)
        *reinterpret_cast<f4 *>(red + row + eb * 16 + 4 * lgrp()) = acc;
    else if (lgrp() == 0)
        red[row + C::D] = acc[0];
}

template <typename T> __device__ __forceinline__ void store4(T *p, f4 v);
template <> __device__ __forceinline__ void store4<float>(float *p, f4 v) { *reinterpret_cast<f4 *>(p) = v; }
template <> __device__ __forceinline__ void store4<__bf16>(__bf16 *p, f4 v)
{
    bf4 r = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *reinterpret_cast<bf4 *>(p) = r;
}
// Store of an 8- or 16-byte value at byte offset off of base, which the hardware drops
// when it does not lie within the first nbytes: row-bounded output stores without a
// branch, so that the compiler counts them exactly in its memory waits.
template <typename V> __device__ __forceinline__ void bstore(void *base, int nbytes, int off, V x)
{
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, nbytes, 0x00020000);
    if constexpr (sizeof(V) == 8) {
        typedef unsigned int u2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, x), r, off, 0, 0);
    } else {
        static_assert(sizeof(V) == 16, "8- or 16-byte values");
        typedef unsigned int u4 __attribute__((ext_vector_type(4)));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, x), r, off, 0, 0);
    }
}
// Four values as the I/O type, row-bounded as bstore.
template <typename T> __device__ __forceinline__ void bstore4(T *base, int nbytes, int off, f4 v)
{
    if constexpr (sizeof(T) == 2)
        bstore(base, nbytes, off, bf4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]});
    else
        bstore(base, nbytes, off, v);
}

// ----------------------------------------------------------- featmap ---

// phi[r][m] = g(X_r)_m in fp32.  With row_off non-null (FAVOR+ only) the row is
// divided by exp(row_off[r]), row_off[r] = max_m (w_m.x_r - |x_r|^2/2).
// A workgroup walks FEATMAP_TILES tiles of rows with W's fragments held in registers
// and the next tile's rows in flight (one tile per workgroup re-read W from L2 for every
// 32 rows), and each wave writes its features through LDS as whole row segments
// (written straight from the MFMA layout, every store instruction touched 16 rows; the
// kernel is a stream of M fp32 per row: 0.40 -> 0.24 ms at 1M rows, M = 256).
constexpr int FEATMAP_TILES = 8;
template <class C>
__global__ __launch_bounds__(C::NT) void featmap_kernel(const void *Xv, const void *Wv, float *phi, float *row_off,
                                                        long long rows)
{
    typedef typename C::T T;
    __shared__ __align__(16) T xs_[C::XMat::SIZE];
    __shared__ float kn[C::TT];
    __shared__ float qmax[C::NW * C::TT];
    __shared__ __align__(16) float fst[C::NW * C::TT * (C::MW + 4)];
    const typename C::XMat xs(xs_);
    const long long rb = (long long)blockIdx.x * C::TT * FEATMAP_TILES;
    const long long re = min(rows, rb + (long long)C::TT * FEATMAP_TILES);
    Frag<T> wf[C::NFB][C::NEB];
    if constexpr (C::FAVOR) load_wfrag<C>(wf, Wv);
    const float lns = 0.5f * __logf((float)C::M);
    typename C::Tile rx;
    rx.load((const T *)Xv + rb * C::D, (int)min((long long)C::TT, re - rb));
    for (long long r0 = rb; r0 < re; r0 += C::TT) {
        const int nv = (int)min((long long)C::TT, re - r0);
        if constexpr (C::FAVOR)
            rx.store(xs, false, [&](int t, float q) { kn[t] = q; });
        else
            rx.store(xs, false, nullptr);
        __syncthreads();
        if (r0 + C::TT < re) rx.load((const T *)Xv + (r0 + C::TT) * C::D, (int)min((long long)C::TT, re - r0 - C::TT));
        f4 ph[C::NFB][C::NTB];
        feat_T<C>(ph, xs, wf);
        if constexpr (C::FAVOR) {
#pragma unroll
            for (int tb = 0; tb < C::NTB; ++tb)
#pragma unroll
                for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) ph[fb][tb][j] -= 0.5f * kn[tb * 16 + lcol()];
            if (row_off) q_partial_max<C>(ph, qmax);
            __syncthreads();
#pragma unroll
            for (int tb = 0; tb < C::NTB; ++tb) {
                const int t = tb * 16 + lcol();
                float off = 0.f;
                if (row_off) {
                    off = qmax[t];
#pragma unroll
                    for (int w = 1; w < C::NW; ++w) off = fmaxf(off, qmax[w * C::TT + t]);
                    if (wave_id() == 0 && lgrp() == 0 && t < nv) row_off[r0 + t] = off;
                }
                const float o2 = -(off + lns) * LOG2E;
#pragma unroll
                for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) ph[fb][tb][j] = __builtin_amdgcn_exp2f(fmaf(ph[fb][tb][j], LOG2E, o2));
            }
        }
        // through this wave's LDS rows, so that each store instruction writes whole
        // MW-feature row segments of 64 / (MW / 4) rows
        {
            float *wb = fst + wave_id() * C::TT * (C::MW + 4);
#pragma unroll
            for (int tb = 0; tb < C::NTB; ++tb)
#pragma unroll
                for (int fb = 0; fb < C::NFB; ++fb)
                    *reinterpret_cast<f4 *>(wb + (tb * 16 + lcol()) * (C::MW + 4) + fb * 16 + 4 * lgrp()) = ph[fb][tb];
            wave_lds_fence();
            constexpr int LPR = C::MW / 4;  // lanes per row
            constexpr int RPI = 64 / LPR;   // rows per instruction
#pragma unroll
            for (int i = 0; i < C::TT / RPI; ++i) {
                const int t = i * RPI + lane_id() / LPR, cc = (lane_id() % LPR) * 4;
                const f4 v = *reinterpret_cast<const f4 *>(wb + t * (C::MW + 4) + cc);
                if (t < nv) *reinterpret_cast<f4 *>(phi + (size_t)(r0 + t) * C::M + wave_id() * C::MW + cc) = v;
            }
        }
        __syncthreads();  // xs, kn and qmax are rewritten for the next tile
    }
}

// -------------------------------------------------------------- chunk ---

struct ChunkGeom {
    int nl;          // chunk index within the window
    int bh;          // head
    long long row0;  // first row of the chunk
    int len;         // rows in the chunk
    size_t hb;       // element offset of the chunk's first row in a [B,H,L,D] tensor
};
template <class C> __device__ __forceinline__ ChunkGeom chunk_geom(const ChunkArgs &a)
{
    ChunkGeom g;
    g.nl = blockIdx.x;
    g.bh = blockIdx.y;
    g.row0 = (long long)(a.n0 + g.nl) * a.c;
    g.len = (int)min((long long)a.c, a.L - g.row0);
    g.hb = (size_t)g.bh * (size_t)a.L * C::D + (size_t)g.row0 * C::D;
    return g;
}
template <class C> __device__ __forceinline__ float *slot_ptr(float *base, const ChunkArgs &a, int bh, int s)
{
    return base + ((size_t)bh * (a.P + 1) + s) * C::SZ;
}

// Stage a K tile: rows past the chunk give g = 0 (kn2 = +inf for FAVOR+, -inf
// inputs for elu+1).
template <class C>
__device__ __forceinline__ void store_k_tile(typename C::Tile &rk, const typename C::XMat &xk, float *kn2, int nv,
                                             float koff)
{
    if constexpr (C::FAVOR) {
        rk.store(xk, false, KnormFn<C>{kn2, nv, koff});
    } else {
        rk.fill_invalid(nv, -__builtin_inff());
        rk.store(xk, false, nullptr);
    }
}
// Stage a V tile and its auxiliary column of ones (zero past the chunk).
template <class C>
__device__ __forceinline__ void store_v_tile(const typename C::Tile &rv, const AugTile<C> &V, int nv)
{
    rv.store(V.x, false, nullptr);
    if (threadIdx.x < C::TT) V.set_aux(threadIdx.x, threadIdx.x < nv ? 1.f : 0.f);
}

// State block of a wave (rows m, cols e) from a slot stored [e][m] (row D = S);
// the auxiliary block holds S in column D.
template <class C> __device__ __forceinline__ void load_state_T(f4 (&rt)[C::NFB][C::NEA], const float *slot)
{
    const int w = wave_id();
#pragma unroll
    for (int fb = 0; fb < C::NFB; ++fb) {
        const int m = w * C::MW + fb * 16 + 4 * lgrp();
#pragma unroll
        for (int eb = 0; eb < C::NEB; ++eb)
            rt[fb][eb] = *reinterpret_cast<const f4 *>(slot + (size_t)(eb * 16 + lcol()) * C::M + m);
        rt[fb][C::NEB] = lcol() == 0 ? *reinterpret_cast<const f4 *>(slot + (size_t)C::D * C::M + m) : f4zero();
    }
}
template <class C> __device__ __forceinline__ void store_state_T(float *slot, const f4 (&rt)[C::NFB][C::NEA])
{
    const int w = wave_id();
#pragma unroll
    for (int fb = 0; fb < C::NFB; ++fb) {
        const int m = w * C::MW + fb * 16 + 4 * lgrp();
#pragma unroll
        for (int eb = 0; eb < C::NEB; ++eb)
            *reinterpret_cast<f4 *>(slot + (size_t)(eb * 16 + lcol()) * C::M + m) = rt[fb][eb];
        if (lcol() == 0) *reinterpret_cast<f4 *>(slot + (size_t)C::D * C::M + m) = rt[fb][C::NEB];
    }
}

// state_kernel: slot[n+1] = (dR_n, dS_n) of chunk n (R part stored [e][m]).
template <class C> struct StateSmem {
    typedef typename C::T T;
    __align__(16) T xk[C::XMat::SIZE];
    __align__(16) T xv[C::XMat::SIZE];
    __align__(16) T xva[C::AuxMat::SIZE];
    float kn2[C::TT];
};
template <class C>
__global__ __launch_bounds__(C::NT, waves_per_simd(sizeof(StateSmem<C>), C::NW)) void state_kernel(ChunkArgs a)
{
    typedef typename C::T T;
    constexpr int NFB = C::NFB, NEA = C::NEA, NTB = C::NTB, TT = C::TT;
    __shared__ StateSmem<C> sm;
    float *kn2 = sm.kn2;
    const typename C::XMat xk(sm.xk);
    const AugTile<C> V(sm.xv, sm.xva);
    const ChunkGeom G = chunk_geom<C>(a);
    const T *Kp = (const T *)a.K + G.hb, *Vp = (const T *)a.V + G.hb;
    Frag<T> wf[NFB][C::NEB];
    if constexpr (C::FAVOR) load_wfrag<C>(wf, a.W);
    const float koff = key_off<C>(a);
    f4 rt[NFB][NEA];
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
        for (int eb = 0; eb < NEA; ++eb) rt[fb][eb] = f4zero();
    // two tiles in flight: this kernel's per-tile work is short, so one tile of
    // prefetch left part of the load latency exposed
    typename C::Tile rk[2], rv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        if (i * TT < G.len) {
            rk[i].load(Kp + (size_t)(i * TT) * C::D, min(TT, G.len - i * TT));
            rv[i].load(Vp + (size_t)(i * TT) * C::D, min(TT, G.len - i * TT));
        }
    for (int t00 = 0; t00 < G.len; t00 += 2 * TT) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t0 = t00 + i * TT;
            if (t0 >= G.len) break;
            const int nv = min(TT, G.len - t0);
            store_k_tile<C>(rk[i], xk, kn2, nv, koff);
            store_v_tile<C>(rv[i], V, nv);
            __syncthreads();
            if (t0 + 2 * TT < G.len) {  // prefetch two tiles ahead
                const int nv2 = min(TT, G.len - t0 - 2 * TT);
                rk[i].load(Kp + (size_t)(t0 + 2 * TT) * C::D, nv2);
                rv[i].load(Vp + (size_t)(t0 + 2 * TT) * C::D, nv2);
            }
            f4 pk[NTB][NFB];
            feat_S<C>(pk, xk, wf);
            k_finish_S<C>(pk, kn2);
            Frag<T> fk[NTB][NFB];
            to_frags<C>(fk, pk);
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
                for (int eb = 0; eb < NEA; ++eb)
                    mma_range<T>(rt[fb][eb], 0, NTB, [&](int tb) { return fk[tb][fb]; },
                                 [&](int tb) { return V.fr(eb, tb * 16); });
            __syncthreads();
        }
    }
    store_state_T<C>(slot_ptr<C>(a.slots, a, G.bh, G.nl + 1), rt);
}

// scan_kernel: per-head sweep over the window's chunk slots (4 floats of the
// (d+1) x M state per element; carryR [BH][d*M], carryS [BH][M]), with the
// running state ("carry") kept in fp64 so that no precision is lost across many
// chunks or windows.  slot[0] = state entering the window's first chunk; slot[n+1]
// holds chunk n's contribution on entry and, for modes 0-2, leaves with:
//   MODE 0  forward prefix:   slot[n+1] = carry + sum_{n' <= n} contribution; carry = the last
//   MODE 1  backward window:  start = carry - sum of the window's contributions (the
//                             reversal of Subsection 3.3 at window granularity), then as
//                             MODE 0 from start; carry = start
//   MODE 2  gradient suffix:  slot[n+1] = carry + sum_{n' > n} contribution, slot[0] = all;
//                             carry = slot[0]
//   MODE 3  accumulate:       carry += sum of the window's contributions (slots untouched)
// The np chunks are cut into G segments (G a power of two <= 32, chosen by the host
// for parallelism): a workgroup holds G segments x 256/G elements; each thread sums its
// segment, the segment totals are exchanged through LDS, and each thread then sweeps
// its segment starting from the carry plus the totals of the segments before it
// (after it, for the suffix).
// SCAN_KEEP: segments of at most that many slots are read once, held in registers from
// the totals pass to the sweep (KEEP, for when there is a totals pass); the variant
// without keeps its registers low for the single sweep.
constexpr int SCAN_KEEP = 32;
template <int MODE, bool KEEP>
__global__ __launch_bounds__(256) void scan_kernel(float *slots, double *carryR, double *carryS, int DM, int M, int P,
                                                   int np, int G)
{
    __shared__ double tot[256][4];
    const int SZ = DM + M;
    const int E = 256 / G;                     // elements per workgroup
    const int g = threadIdx.x / E, el = threadIdx.x % E;
    const int k = (blockIdx.x * E + el) * 4;   // first float of this thread's element
    const bool active = k < SZ;
    const int bh = blockIdx.y;
    const int sl = (np + G - 1) / G;
    const int na = min(np, g * sl), nb = min(np, na + sl);
    float *base = slots + (size_t)bh * (P + 1) * SZ + (active ? k : 0);
    double *cp = !active ? nullptr : k < DM ? carryR + (size_t)bh * DM + k : carryS + (size_t)bh * M + (k - DM);
    auto slot = [&](int i) { return reinterpret_cast<f4 *>(base + (size_t)i * SZ); };
    auto put = [&](int i, const double *v) { *slot(i) = f4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]}; };
    // segment totals: needed by the window-start and accumulate modes, and by every
    // mode when the chunks are split over several segments
    const bool totals = MODE == 1 || MODE == 3 || G > 1;
    // (the sums keep their order either way)
    const bool keep = KEEP && totals && sl <= SCAN_KEEP;
    f4 buf[KEEP ? SCAN_KEEP : 1];
    double cur[4] = {0.0, 0.0, 0.0, 0.0}, seg[4] = {0.0, 0.0, 0.0, 0.0};
    if (active) {
#pragma unroll
        for (int j = 0; j < 4; ++j) cur[j] = cp[j];
        if (keep) {
#pragma unroll
            for (int u = 0; u < (KEEP ? SCAN_KEEP : 0); ++u)
                if (na + u < nb) buf[u] = *slot(na + u + 1);
#pragma unroll
            for (int u = 0; u < (KEEP ? SCAN_KEEP : 0); ++u)
                if (na + u < nb)
#pragma unroll
                    for (int j = 0; j < 4; ++j) seg[j] += (double)buf[u][j];
        } else {
            for (int n = na; totals && n < nb; ++n) {
                const f4 dl = *slot(n + 1);
#pragma unroll
                for (int j = 0; j < 4; ++j) seg[j] += (double)dl[j];
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) tot[threadIdx.x][j] = seg[j];
    __syncthreads();
    // totals of the segments before this one, after it, and of all of them (each a sum
    // of its own segments, never a difference, so that one non-finite contribution
    // reaches only the slices whose prefix or suffix contains it)
    double before[4] = {0.0, 0.0, 0.0, 0.0}, after[4] = {0.0, 0.0, 0.0, 0.0}, all[4] = {0.0, 0.0, 0.0, 0.0};
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double t = tot[h * E + el][j];
            all[j] += t;
            if (h < g) before[j] += t;
            if (h > g) after[j] += t;
        }
    if (!active) return;
    const bool last = g == G - 1;
    if (MODE == 3) {
        if (last)
#pragma unroll
            for (int j = 0; j < 4; ++j) cp[j] = cur[j] + all[j];
        return;
    }
    if (MODE == 0 || MODE == 1) {
        double start[4], run[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            start[j] = MODE == 1 ? cur[j] - all[j] : cur[j];
            run[j] = start[j] + before[j];
        }
        if (g == 0) put(0, start);
        if (keep) {
#pragma unroll
            for (int u = 0; u < (KEEP ? SCAN_KEEP : 0); ++u)
                if (na + u < nb) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) run[j] += (double)buf[u][j];
                    put(na + u + 1, run);
                }
        } else {
            for (int n = na; n < nb; ++n) {
                const f4 dl = *slot(n + 1);
#pragma unroll
                for (int j = 0; j < 4; ++j) run[j] += (double)dl[j];
                put(n + 1, run);
            }
        }
        if (last)
#pragma unroll
            for (int j = 0; j < 4; ++j) cp[j] = MODE == 0 ? run[j] : start[j];
    } else {  // MODE 2
        double run[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) run[j] = cur[j] + after[j];
        if (keep) {
#pragma unroll
            for (int u = (KEEP ? SCAN_KEEP : 0) - 1; u >= 0; --u)
                if (na + u < nb) {
                    put(na + u + 1, run);
#pragma unroll
                    for (int j = 0; j < 4; ++j) run[j] += (double)buf[u][j];
                }
        } else {
            for (int n = nb - 1; n >= na; --n) {
                const f4 dl = *slot(n + 1);
                put(n + 1, run);
#pragma unroll
                for (int j = 0; j < 4; ++j) run[j] += (double)dl[j];
            }
        }
        if (g == 0) {
            put(0, run);
#pragma unroll
            for (int j = 0; j < 4; ++j) cp[j] = run[j];
        }
    }
}

// LDS of the chunk kernels that evaluate a chunk's forward.  RED: per-wave fp32
// rows for the cross-wave sum of the numerators (else two floats per row and wave).
template <class C, bool RED = true> struct FwdSmem {
    typedef typename C::T T;
    __align__(16) T xq[C::XMat::SIZE];
    __align__(16) T xk[C::XMat::SIZE];
    __align__(16) T xv[C::XMat::SIZE];
    __align__(16) T xva[C::AuxMat::SIZE];
    __align__(16) T fk[C::NW * C::FMat::SIZE];
    __align__(16) float red[RED ? C::NW * C::TT * C::LDR : 2 * C::NW * C::TT];
    float qmax[C::NW * C::TT];
    float kn2[C::TT];
};

// Q, K, V tiles of the chunk forward, held in registers between prefetch and use.
template <class C> struct FwdRegs {
    typedef typename C::T T;
    typename C::Tile q, k, v;
    __device__ __forceinline__ void load(const T *Q, const T *K, const T *V, int t0, int len)
    {
        const int nv = min(C::TT, len - t0);
        q.load(Q + (size_t)t0 * C::D, nv);
        k.load(K + (size_t)t0 * C::D, nv);
        v.load(V + (size_t)t0 * C::D, nv);
    }
    template <class SM> __device__ __forceinline__ void store(SM &sm, int nv, float koff)
    {
        q.store(typename C::XMat(sm.xq), false, nullptr);
        store_k_tile<C>(k, typename C::XMat(sm.xk), sm.kn2, nv, koff);
        store_v_tile<C>(v, AugTile<C>(sm.xv, sm.xva), nv);
    }
};

// One tile of the chunk forward, shared by fwd_kernel and stats_kernel: hands
// this wave's partial numerator^T blocks (rows e, cols t; the auxiliary block's
// first row is the denominator), scaled by the wave's own query offset (recorded in
// sm.qmax), to emit(eb, tb, acc); leaves g(Q) of this wave's features (rows m,
// cols t) in pq and g(K) in the wave's feature buffer (rows t, cols m).
template <class C, class SM, class EMIT>
__device__ __forceinline__ void fwd_tile(SM &sm, const Frag<typename C::T> (&wf)[C::NFB][C::NEB],
                                         const f4 (&rt)[C::NFB][C::NEA], f4 (&pq)[C::NFB][C::NTB], EMIT emit)
{
    typedef typename C::T T;
    constexpr int NFB = C::NFB, NEA = C::NEA, NTB = C::NTB;
    const int g = lgrp(), lc = lcol();
    const typename C::XMat xq(sm.xq), xk(sm.xk);
    const AugTile<C> V(sm.xv, sm.xva);
    const typename C::FMat Fk(sm.fk + wave_id() * C::FMat::SIZE);
    f4 pkT[NFB][NTB];
    feat_T<C>(pq, xq, wf);
    feat_T<C>(pkT, xk, wf);
    q_wave_finish<C>(pq, sm.qmax);
    k_finish_T<C>(pkT, sm.kn2);
    Frag<T> fq[NFB][NTB], fkT[NFB][NTB];
    to_frags<C>(fq, pq);
    to_frags<C>(fkT, pkT);
    put_feature_frags<C>(Fk, fkT);
    // P^T blocks (rows s, cols t) over this wave's features; the blocks above the
    // diagonal (s-block > t-block) are zero
    Frag<T> pt[NTB][NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
        for (int sb = 0; sb < NTB; ++sb) {
            if (sb > tb) {
                pt[sb][tb] = cfrag<T>(f4zero());
                continue;
            }
            f4 acc = f4zero();
            mma_range<T>(acc, 0, NFB, [&](int kb) { return fkT[kb][sb]; }, [&](int kb) { return fq[kb][tb]; });
            if (sb == tb)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (4 * g + j > lc) acc[j] = 0.f;
            pt[sb][tb] = cfrag<T>(acc);
        }
    // partial numerators^T (rows e, cols t; e = D is the denominator): V^T P^T + R g(Q)^T.
    // The product with P^T runs over all s-blocks of the tile, the zero ones included:
    // the V operand pairs then are the same for every t-block, and no block goes
    // through a zero-padded product
#pragma unroll
    for (int eb = 0; eb < NEA; ++eb)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            f4 acc = f4zero();
            mma_range<T>(acc, 0, NTB, [&](int sb) { return V.fr(eb, sb * 16); }, [&](int sb) { return pt[sb][tb]; });
            mma_range<T>(acc, 0, NFB, [&](int fb) { return cfrag<T>(rt[fb][eb]); }, [&](int fb) { return fq[fb][tb]; });
            emit(eb, tb, acc);
        }
}

// State update after a tile: [R^T | S] += g(K)^T [V | 1] over this wave's features.
template <class C, class SM> __device__ __forceinline__ void state_update_T(SM &sm, f4 (&rt)[C::NFB][C::NEA])
{
    typedef typename C::T T;
    const AugTile<C> V(sm.xv, sm.xva);
    const typename C::FMat Fk(sm.fk + wave_id() * C::FMat::SIZE);
#pragma unroll
    for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
        for (int eb = 0; eb < C::NEA; ++eb)
            mma_range<T>(rt[fb][eb], 0, C::NTB, [&](int tb) { return Fk.frag_r(fb * 16, tb * 16); },
                         [&](int tb) { return V.fr(eb, tb * 16); });
}

// fwd_kernel: Y of one chunk from its entry state slot[n].
template <class C>
__global__ __launch_bounds__(C::NT, waves_per_simd(sizeof(FwdSmem<C>), C::NW)) void fwd_kernel(ChunkArgs a)
{
    typedef typename C::T T;
    constexpr int NFB = C::NFB, NEA = C::NEA, NTB = C::NTB, TT = C::TT;
    __shared__ FwdSmem<C> sm;
    const ChunkGeom G = chunk_geom<C>(a);
    const T *Q = (const T *)a.Q + G.hb, *K = (const T *)a.K + G.hb, *V = (const T *)a.V + G.hb;
    T *Y = (T *)a.out0 + G.hb;
    // per-row statistics for the backward: 1/den at the common query offset, and that offset
    float *rs = a.rstat ? a.rstat + ((size_t)G.bh * a.L + G.row0) * 2 : nullptr;
    Frag<T> wf[NFB][C::NEB];
    if constexpr (C::FAVOR) load_wfrag<C>(wf, a.W);
    const float koff = key_off<C>(a);
    f4 rt[NFB][NEA];
    load_state_T<C>(rt, slot_ptr<C>(a.slots, a, G.bh, G.nl));
    FwdRegs<C> rg;
    // Y (and the row records) of a tile, held in registers as stored, are written at the
    // start of the next tile, after the wait for that tile's inputs (a wait for a load
    // also waits for every store issued before it): fwd 1.048 -> 0.986 ms on 1M tokens x
    // 8 heads, 0.226 -> 0.212 ms for elu+1 at d = 128, 0.275 -> 0.272 ms at the 16K-token,
    // 64-head shape
    constexpr int Q4 = C::D / 4, YI = (TT * Q4 + C::NT - 1) / C::NT;
    typedef std::conditional_t<sizeof(T) == 2, bf4, f4> YV;
    YV yv[YI];
    float2 yr[YI];
    int pt0 = -1, pnv = 0;
    auto store_y = [&]() {
#pragma unroll
        for (int k = 0; k < YI; ++k) {
            const int v = threadIdx.x + k * C::NT, t = v / Q4, e = (v % Q4) * 4;
            const int ny = pnv * C::D * (int)sizeof(T), nr = pnv * 8;
            const bool in = v < TT * Q4;
            bstore(Y + (size_t)pt0 * C::D, ny, in ? (t * C::D + e) * (int)sizeof(T) : ny, yv[k]);
            if (rs) bstore(rs + (size_t)pt0 * 2, nr, in && e == 0 ? t * 8 : nr, yr[k]);
        }
    };
    rg.load(Q, K, V, 0, G.len);
    // The phases that end a tile (the reduction of Y, then the state update) run at raised
    // wave priority, so that the other workgroup on the compute unit fills their gaps rather
    // than delaying them: fwd 0.272 -> 0.267 ms at the 16K-token, 64-head shape, 1.00 ->
    // 0.98 ms on 1M tokens x 8 heads (M = 64); no change for elu+1 or fp32.
    for (int t0 = 0; t0 < G.len; t0 += TT) {
        const int nv = min(TT, G.len - t0);
        __builtin_amdgcn_s_setprio(0);
        rg.store(sm, nv, koff);
        if (pt0 >= 0) store_y();
        __syncthreads();
        if (t0 + TT < G.len) rg.load(Q, K, V, t0 + TT, G.len);
        f4 pq[NFB][NTB];
        fwd_tile<C>(sm, wf, rt, pq, [&](int eb, int tb, f4 acc) { put_red<C>(sm.red, eb, tb, acc); });
        __syncthreads();
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int k = 0; k < YI; ++k) {
            const int v = threadIdx.x + k * C::NT, t = v / Q4, e = (v % Q4) * 4;
            if (v < TT * Q4) {
                float sc[C::NW], moff;
                wave_scales<C>(sm.qmax, t, sc, &moff);
                f4 sum = f4zero();
                float den = 0.f;
#pragma unroll
                for (int w = 0; w < C::NW; ++w) {
                    sum += *reinterpret_cast<const f4 *>(sm.red + (w * TT + t) * C::LDR + e) * sc[w];
                    den += sm.red[(w * TT + t) * C::LDR + C::D] * sc[w];
                }
                const float inv = 1.f / den;
                const f4 y = sum * inv;
                if constexpr (sizeof(T) == 2)
                    yv[k] = YV{(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
                else
                    yv[k] = y;
                yr[k] = make_float2(inv, moff);
            }
        }
        pt0 = t0;
        pnv = nv;
        __builtin_amdgcn_s_setprio(1);
        state_update_T<C>(sm, rt);
        __syncthreads();
    }
    store_y();
}

}  // namespace slim
