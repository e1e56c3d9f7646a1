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
// outputs (numerators, dQ, dK, dV) across waves through LDS.
//
// Kernels (all launched on a grid (chunks in window, B*H)):
//   featmap_kernel : standalone g(X), optional per-row max offset.
//   state_kernel   : dR_n = sum_{rows of chunk n} V g(K)^T, dS_n = sum g(K).
//   scan_kernel    : per-head sequential sweep over the window's chunk states
//                    (forward prefix, reverse subtraction, gradient suffix sum).
//   fwd_kernel     : Y for a chunk from its entry state.
//   stats_kernel   : backward pass 1: recompute the chunk forward, emit per-row
//                    1/den and dden = -(dY.Y)/den, and the chunk's gradient
//                    contribution to its entry state: dG_n = sum dNum g(Q)^T.
//   bwdq_kernel    : dQ (forward tile order, entry state R).
//   bwdkv_kernel   : dK, dV (reverse tile order, gradient state dR).
#pragma once
#include "slim_device.h"

namespace slim {

struct ChunkArgs {
    const void *Q, *K, *V, *W, *dY;
    void *out0, *out1, *out2;  // fwd: Y | bwdq: dQ | bwdkv: dK, dV
    float *slots;              // [BH][P+1][(D+1)*M]  state slots (R rows, then S)
    float *gslots;             // [BH][P+1][(D+1)*M]  gradient-state slots
    float *stats;              // [BH][P][c][2]       per-row (1/den, dden)
    long long L;
    int c;   // chunk length
    int n0;  // first chunk of the window
    int P;   // window capacity (slot stride)
};

template <typename T_, int D_, int M_, int FEAT_, int TT_, int MW_ = 32> struct KCfg {
    typedef T_ T;
    static constexpr int D = D_, M = M_, FEAT = FEAT_, TT = TT_;
    static constexpr int MW = M >= MW_ ? MW_ : M;  // features per wave
    static constexpr int NW = M / MW;            // waves per workgroup
    static constexpr int NT = NW * 64;
    static constexpr int NFB = MW / 16;
    static constexpr int NEB = D / 16;
    static constexpr int NTB = TT / 16;
    // LDS row strides: 4 elements of padding make the rows of a 16-row operand
    // read land in distinct banks (stride = 8 bytes mod 128 for bf16, 16 for fp32).
    static constexpr int LDX = D + 4;   // [TT][D] tiles
    static constexpr int LDT = TT + 4;  // [D][TT] transposed tiles
    static constexpr int LDR = D + 4;   // fp32 reduction rows
    static constexpr int SZ = (D + 1) * M;
    static constexpr bool FAVOR = FEAT == FEAT_FAVOR;
    typedef TileRegs<T, D, TT, NT> Tile;
    static_assert(FEAT == FEAT_FAVOR || D == M, "elu+1 needs M == d");
    static_assert(MW % 16 == 0 && D % 16 == 0 && TT % 16 == 0, "block sizes");
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
// (free index e, contraction over this wave's features).
template <class C>
__device__ __forceinline__ void load_wtfrag(Frag<typename C::T> (&wt)[C::NEB][C::NFB], const void *Wv)
{
    typedef typename C::T T;
    const T *W = (const T *)Wv;
    const int w = wave_id();
#pragma unroll
    for (int eb = 0; eb < C::NEB; ++eb)
#pragma unroll
        for (int fb = 0; fb < C::NFB; ++fb) {
            Frag<T> f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                f.v[j] = W[(size_t)(w * C::MW + fb * 16 + 4 * lgrp() + j) * C::D + eb * 16 + lcol()];
            wt[eb][fb] = f;
        }
}

// Feature blocks in "transposed" orientation: ph[fb][tb] has rows m = w*MW + fb*16 + 4g + j
// and columns t = tb*16 + i%16.  FAVOR+: the raw projection w_m . x_t.  elu+1: g itself.
template <class C>
__device__ __forceinline__ void feat_T(f4 (&ph)[C::NFB][C::NTB], const typename C::T *xs,
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
                             [&](int kb) { return lds_frag<T>(xs, C::LDX, tb * 16, kb * 16); });
                ph[fb][tb] = acc;
            } else {
                f4 x = frag_to_f4<T>(lds_frag<T>(xs, C::LDX, tb * 16, wave_id() * C::MW + fb * 16));
                ph[fb][tb] = f4{elu1(x[0]), elu1(x[1]), elu1(x[2]), elu1(x[3])};
            }
        }
}

// Feature blocks in "token" orientation: ph[tb][fb] has rows t = tb*16 + 4g + j and
// columns m = w*MW + fb*16 + i%16.  elu+1 reads the transposed tile xt[D][TT].
template <class C>
__device__ __forceinline__ void feat_S(f4 (&ph)[C::NTB][C::NFB], const typename C::T *xs, const typename C::T *xt,
                                       const Frag<typename C::T> (&wf)[C::NFB][C::NEB])
{
    typedef typename C::T T;
#pragma unroll
    for (int tb = 0; tb < C::NTB; ++tb)
#pragma unroll
        for (int fb = 0; fb < C::NFB; ++fb) {
            if constexpr (C::FAVOR) {
                f4 acc = f4zero();
                mma_range<T>(acc, 0, C::NEB, [&](int kb) { return lds_frag<T>(xs, C::LDX, tb * 16, kb * 16); },
                             [&](int kb) { return wf[fb][kb]; });
                ph[tb][fb] = acc;
            } else {
                f4 x = frag_to_f4<T>(lds_frag<T>(xt, C::LDT, wave_id() * C::MW + fb * 16, tb * 16));
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
template <class C> __device__ __forceinline__ float q_offset(const float *qmax, int t)
{
    float m = qmax[t];
#pragma unroll
    for (int w = 1; w < C::NW; ++w) m = fmaxf(m, qmax[w * C::TT + t]);
    return m;
}

// g(Q) up to a per-row positive factor: exp(w_m.q_t - max_m' w_m'.q_t).  The factor
// cancels in Y and in dQ (Y is homogeneous of degree 0 in each g(Q_l)).
template <class C> __device__ __forceinline__ void q_finish_T(f4 (&ph)[C::NFB][C::NTB], const float *qmax)
{
    if constexpr (C::FAVOR) {
#pragma unroll
        for (int tb = 0; tb < C::NTB; ++tb) {
            const float off = q_offset<C>(qmax, tb * 16 + lcol());
#pragma unroll
            for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
                for (int j = 0; j < 4; ++j) ph[fb][tb][j] = fast_exp(ph[fb][tb][j] - off);
        }
    }
}
template <class C> __device__ __forceinline__ void q_finish_S(f4 (&ph)[C::NTB][C::NFB], const float *qmax)
{
    if constexpr (C::FAVOR) {
#pragma unroll
        for (int tb = 0; tb < C::NTB; ++tb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float off = q_offset<C>(qmax, tb * 16 + 4 * lgrp() + j);
#pragma unroll
                for (int fb = 0; fb < C::NFB; ++fb) ph[tb][fb][j] = fast_exp(ph[tb][fb][j] - off);
            }
    }
}

// g(K) exactly: exp(w_m.k_t - |k_t|^2/2) / sqrt(M) (FAVOR+), zero for rows t >= nv.
template <class C>
__device__ __forceinline__ void k_finish_T(f4 (&ph)[C::NFB][C::NTB], const float *kn, int nv)
{
    const float lns = 0.5f * __logf((float)C::M);
#pragma unroll
    for (int tb = 0; tb < C::NTB; ++tb) {
        const int t = tb * 16 + lcol();
        const bool ok = t < nv;
        const float off = C::FAVOR ? 0.5f * kn[t] + lns : 0.f;
#pragma unroll
        for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ph[fb][tb][j] = !ok ? 0.f : (C::FAVOR ? fast_exp(ph[fb][tb][j] - off) : ph[fb][tb][j]);
    }
}
template <class C>
__device__ __forceinline__ void k_finish_S(f4 (&ph)[C::NTB][C::NFB], const float *kn, int nv)
{
    const float lns = 0.5f * __logf((float)C::M);
#pragma unroll
    for (int tb = 0; tb < C::NTB; ++tb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = tb * 16 + 4 * lgrp() + j;
            const bool ok = t < nv;
            const float off = C::FAVOR ? 0.5f * kn[t] + lns : 0.f;
#pragma unroll
            for (int fb = 0; fb < C::NFB; ++fb)
                ph[tb][fb][j] = !ok ? 0.f : (C::FAVOR ? fast_exp(ph[tb][fb][j] - off) : ph[tb][fb][j]);
        }
}

template <class C, int A, int B>
__device__ __forceinline__ void to_frags(Frag<typename C::T> (&f)[A][B], const f4 (&c)[A][B])
{
#pragma unroll
    for (int a = 0; a < A; ++a)
#pragma unroll
        for (int b = 0; b < B; ++b) f[a][b] = cfrag<typename C::T>(c[a][b]);
}

// Sum the NW per-wave fp32 partials red[w][t][e] for tile rows, divide by den (if
// given) and hand (t, e..e+3, value) to `emit` for every valid row.
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

template <typename T> __device__ __forceinline__ void store4(T *p, f4 v);
template <> __device__ __forceinline__ void store4<float>(float *p, f4 v) { *reinterpret_cast<f4 *>(p) = v; }
template <> __device__ __forceinline__ void store4<__bf16>(__bf16 *p, f4 v)
{
    bf4 r = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *reinterpret_cast<bf4 *>(p) = r;
}
template <typename T> __device__ __forceinline__ f4 load4(const T *p);
template <> __device__ __forceinline__ f4 load4<float>(const float *p) { return *reinterpret_cast<const f4 *>(p); }
template <> __device__ __forceinline__ f4 load4<__bf16>(const __bf16 *p)
{
    bf4 r = *reinterpret_cast<const bf4 *>(p);
    return f4{(float)r[0], (float)r[1], (float)r[2], (float)r[3]};
}

// ----------------------------------------------------------- featmap ---

// phi[r][m] = g(X_r)_m in fp32.  With row_off non-null (FAVOR+ only) the row is
// divided by exp(row_off[r]), row_off[r] = max_m (w_m.x_r - |x_r|^2/2).
template <class C>
__global__ __launch_bounds__(C::NT) void featmap_kernel(const void *Xv, const void *Wv, float *phi, float *row_off,
                                                        long long rows)
{
    typedef typename C::T T;
    __shared__ __align__(16) T xs[C::TT * C::LDX];
    __shared__ float kn[C::TT];
    __shared__ float qmax[C::NW * C::TT];
    const long long r0 = (long long)blockIdx.x * C::TT;
    const int nv = (int)min((long long)C::TT, rows - r0);
    const T *X = (const T *)Xv + r0 * C::D;
    Frag<T> wf[C::NFB][C::NEB];
    if constexpr (C::FAVOR) load_wfrag<C>(wf, Wv);
    {
        typename C::Tile rx;
        rx.load(X, nv);
        rx.store(xs, C::LDX, nullptr, 0, false, C::FAVOR ? kn : nullptr);
    }
    __syncthreads();
    f4 ph[C::NFB][C::NTB];
    feat_T<C>(ph, xs, wf);
    const float lns = 0.5f * __logf((float)C::M);
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
            const float off = row_off ? q_offset<C>(qmax, t) : 0.f;
            if (row_off && wave_id() == 0 && lgrp() == 0 && t < nv) row_off[r0 + t] = off;
#pragma unroll
            for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
                for (int j = 0; j < 4; ++j) ph[fb][tb][j] = fast_exp(ph[fb][tb][j] - off - lns);
        }
    }
#pragma unroll
    for (int tb = 0; tb < C::NTB; ++tb) {
        const int t = tb * 16 + lcol();
        if (t < nv)
#pragma unroll
            for (int fb = 0; fb < C::NFB; ++fb)
                *reinterpret_cast<f4 *>(phi + (size_t)(r0 + t) * C::M + wave_id() * C::MW + fb * 16 + 4 * lgrp()) =
                    ph[fb][tb];
    }
}

// -------------------------------------------------------------- chunk ---

struct ChunkGeom {
    int nl;          // chunk index within the window
    int bh;          // head
    long long row0;  // first row of the chunk
    int len;         // rows in the chunk
    size_t hb;       // element offset of the head in a [B,H,L,D] tensor
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

// state_kernel: slot[n+1] = (dR_n, dS_n) of chunk n (R part stored [e][m]).
template <class C> __global__ __launch_bounds__(C::NT) void state_kernel(ChunkArgs a)
{
    typedef typename C::T T;
    constexpr int NFB = C::NFB, NEB = C::NEB, NTB = C::NTB, TT = C::TT;
    __shared__ __align__(16) T xk[TT * C::LDX];
    __shared__ __align__(16) T kt[C::FAVOR ? 8 : C::D * C::LDT];
    __shared__ __align__(16) T vt[C::D * C::LDT];
    __shared__ float kn[TT];
    const ChunkGeom G = chunk_geom<C>(a);
    const int w = wave_id(), g = lgrp(), lc = lcol();
    const T *K = (const T *)a.K + G.hb, *V = (const T *)a.V + G.hb;
    Frag<T> wf[NFB][NEB];
    if constexpr (C::FAVOR) load_wfrag<C>(wf, a.W);
    f4 rt[NFB][NEB];
    float sacc[NFB];
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) {
        sacc[fb] = 0.f;
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb) rt[fb][eb] = f4zero();
    }
    typename C::Tile rk, rv;
    rk.load(K, min(TT, G.len));
    rv.load(V, min(TT, G.len));
    for (int t0 = 0; t0 < G.len; t0 += TT) {
        const int nv = min(TT, G.len - t0);
        rk.store(xk, C::LDX, C::FAVOR ? nullptr : kt, C::LDT, false, C::FAVOR ? kn : nullptr);
        rv.store(nullptr, 0, vt, C::LDT, false, nullptr);
        __syncthreads();
        if (t0 + TT < G.len) {  // prefetch the next tile while this one is computed
            const int nv1 = min(TT, G.len - t0 - TT);
            rk.load(K + (size_t)(t0 + TT) * C::D, nv1);
            rv.load(V + (size_t)(t0 + TT) * C::D, nv1);
        }
        f4 pk[NTB][NFB];
        feat_S<C>(pk, xk, kt, wf);
        k_finish_S<C>(pk, kn, nv);
        Frag<T> fk[NTB][NFB];
        to_frags<C>(fk, pk);
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb) {
#pragma unroll
            for (int eb = 0; eb < NEB; ++eb)
                mma_range<T>(rt[fb][eb], 0, NTB, [&](int tb) { return fk[tb][fb]; },
                             [&](int tb) { return lds_frag<T>(vt, C::LDT, eb * 16, tb * 16); });
            float s = 0.f;
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) s += pk[tb][fb][0] + pk[tb][fb][1] + pk[tb][fb][2] + pk[tb][fb][3];
            sacc[fb] += sum_groups(s);
        }
        __syncthreads();
    }
    float *out = slot_ptr<C>(a.slots, a, G.bh, G.nl + 1);
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) {
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb)
            *reinterpret_cast<f4 *>(out + (size_t)(eb * 16 + lc) * C::M + w * C::MW + fb * 16 + 4 * g) = rt[fb][eb];
        if (g == 0) out[C::D * C::M + w * C::MW + fb * 16 + lc] = sacc[fb];
    }
}

// scan_kernel: sweep the window's chunk slots of one head.  Each thread owns 4
// consecutive floats of the (D+1)*M state.  carryR [BH][D*M], carryS [BH][M].
//   MODE 0 (forward prefix):  slot[0] = carry; slot[n+1] = slot[n] + dR_n; carry = slot[np].
//   MODE 1 (reverse subtract): carry holds the state after the window;
//                              slot[n+1] = state after chunk n, slot[0] = carry = state
//                              before the window (update (19) of the page).
//   MODE 2 (gradient suffix):  carry holds the gradient after the window; slot[n+1] =
//                              gradient w.r.t. the state after chunk n; slot[0] = carry =
//                              gradient w.r.t. the state before the window.
template <int MODE>
__global__ __launch_bounds__(256) void scan_kernel(float *slots, float *carryR, float *carryS, int DM, int M, int P,
                                                   int np)
{
    const int SZ = DM + M;
    const int k = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (k >= SZ) return;
    const int bh = blockIdx.y;
    float *base = slots + (size_t)bh * (P + 1) * SZ + k;
    float *cp = k < DM ? carryR + (size_t)bh * DM + k : carryS + (size_t)bh * M + (k - DM);
    f4 cur = *reinterpret_cast<f4 *>(cp);
    if (MODE == 0) {
        *reinterpret_cast<f4 *>(base) = cur;
        for (int n = 0; n < np; ++n) {
            f4 *p = reinterpret_cast<f4 *>(base + (size_t)(n + 1) * SZ);
            cur += *p;
            *p = cur;
        }
    } else {
        for (int n = np - 1; n >= 0; --n) {
            f4 *p = reinterpret_cast<f4 *>(base + (size_t)(n + 1) * SZ);
            const f4 dlt = *p;
            *p = cur;
            if (MODE == 1) cur -= dlt; else cur += dlt;
        }
        *reinterpret_cast<f4 *>(base) = cur;
    }
    *reinterpret_cast<f4 *>(cp) = cur;
}

// Shared LDS layout of the chunk kernels that evaluate a chunk's forward.
template <class C> struct FwdSmem {
    typedef typename C::T T;
    __align__(16) T xq[C::TT * C::LDX];
    __align__(16) T xk[C::TT * C::LDX];
    __align__(16) T vt[C::D * C::LDT];
    __align__(16) T kt[C::FAVOR ? 8 : C::D * C::LDT];
    __align__(16) T qt[C::FAVOR ? 8 : C::D * C::LDT];
    __align__(16) float red[C::NW * C::TT * C::LDR];
    float redd[C::NW * C::TT];
    float qmax[C::NW * C::TT];
    float kn[C::TT];
    float Sl[C::M];
};

// One tile of the chunk forward shared by fwd_kernel and stats_kernel:
// computes this wave's partial numerator^T / denominator into red/redd (then
// syncs), leaves g(Q) (transposed blocks), g(K) (token blocks) in the outputs.
template <class C>
__device__ __forceinline__ void fwd_tile(FwdSmem<C> &sm, const Frag<typename C::T> (&wf)[C::NFB][C::NEB],
                                         const f4 (&rt)[C::NFB][C::NEB], int nv, f4 (&pq)[C::NFB][C::NTB],
                                         f4 (&pk)[C::NTB][C::NFB])
{
    typedef typename C::T T;
    constexpr int NFB = C::NFB, NEB = C::NEB, NTB = C::NTB, TT = C::TT;
    const int w = wave_id(), g = lgrp(), lc = lcol();
    f4 pkT[NFB][NTB];
    feat_T<C>(pq, sm.xq, wf);
    feat_T<C>(pkT, sm.xk, wf);
    feat_S<C>(pk, sm.xk, sm.kt, wf);
    if constexpr (C::FAVOR) q_partial_max<C>(pq, sm.qmax);
    __syncthreads();
    q_finish_T<C>(pq, sm.qmax);
    k_finish_T<C>(pkT, sm.kn, nv);
    k_finish_S<C>(pk, sm.kn, nv);
    Frag<T> fq[NFB][NTB], fkT[NFB][NTB];
    to_frags<C>(fq, pq);
    to_frags<C>(fkT, pkT);
    // P^T blocks (rows s, cols t), s-block <= t-block, over this wave's features.
    f4 pt[NTB][NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
        for (int sb = 0; sb <= tb; ++sb) {
            f4 acc = f4zero();
            mma_range<T>(acc, 0, NFB, [&](int kb) { return fkT[kb][sb]; }, [&](int kb) { return fq[kb][tb]; });
            if (sb == tb)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (4 * g + j > lc) acc[j] = 0.f;
            pt[sb][tb] = acc;
        }
    // partial denominators (per column t): sum_s P^T[s][t] + g(Q_t) . S (own features)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
        float v = 0.f;
#pragma unroll
        for (int sb = 0; sb <= tb; ++sb) v += pt[sb][tb][0] + pt[sb][tb][1] + pt[sb][tb][2] + pt[sb][tb][3];
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int j = 0; j < 4; ++j) v += pq[fb][tb][j] * sm.Sl[w * C::MW + fb * 16 + 4 * g + j];
        v = sum_groups(v);
        if (g == 0) sm.redd[w * TT + tb * 16 + lc] = v;
    }
    // partial numerators^T (rows e, cols t): V^T P^T + R g(Q)^T
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            f4 acc = f4zero();
            mma_range<T>(acc, 0, tb + 1, [&](int sb) { return lds_frag<T>(sm.vt, C::LDT, eb * 16, sb * 16); },
                         [&](int sb) { return cfrag<T>(pt[sb][tb]); });
            mma_range<T>(acc, 0, NFB, [&](int fb) { return cfrag<T>(rt[fb][eb]); }, [&](int fb) { return fq[fb][tb]; });
            *reinterpret_cast<f4 *>(sm.red + (w * TT + tb * 16 + lc) * C::LDR + eb * 16 + 4 * g) = acc;
        }
    __syncthreads();
}

// State update after a tile: R^T += g(K)^T V, S += sum g(K) (own features).
template <class C>
__device__ __forceinline__ void state_update_T(FwdSmem<C> &sm, f4 (&rt)[C::NFB][C::NEB], const f4 (&pk)[C::NTB][C::NFB])
{
    typedef typename C::T T;
    constexpr int NFB = C::NFB, NEB = C::NEB, NTB = C::NTB;
    Frag<T> fk[NTB][NFB];
    to_frags<C>(fk, pk);
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) {
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb)
            mma_range<T>(rt[fb][eb], 0, NTB, [&](int tb) { return fk[tb][fb]; },
                         [&](int tb) { return lds_frag<T>(sm.vt, C::LDT, eb * 16, tb * 16); });
        float s = 0.f;
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) s += pk[tb][fb][0] + pk[tb][fb][1] + pk[tb][fb][2] + pk[tb][fb][3];
        s = sum_groups(s);
        if (lgrp() == 0) sm.Sl[wave_id() * C::MW + fb * 16 + lcol()] += s;
    }
}

template <class C>
__device__ __forceinline__ void load_state_T(f4 (&rt)[C::NFB][C::NEB], float *Sl, const float *slot)
{
    const int w = wave_id();
#pragma unroll
    for (int fb = 0; fb < C::NFB; ++fb)
#pragma unroll
        for (int eb = 0; eb < C::NEB; ++eb)
            rt[fb][eb] = *reinterpret_cast<const f4 *>(slot + (size_t)(eb * 16 + lcol()) * C::M + w * C::MW + fb * 16 +
                                                        4 * lgrp());
    for (int m = threadIdx.x; m < C::M; m += C::NT) Sl[m] = slot[C::D * C::M + m];
}

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
    __device__ __forceinline__ void store(FwdSmem<C> &sm, bool q_transposed) const
    {
        q.store(sm.xq, C::LDX, (!C::FAVOR && q_transposed) ? sm.qt : nullptr, C::LDT, false, nullptr);
        k.store(sm.xk, C::LDX, C::FAVOR ? nullptr : sm.kt, C::LDT, false, C::FAVOR ? sm.kn : nullptr);
        v.store(nullptr, 0, sm.vt, C::LDT, false, nullptr);
    }
};

// fwd_kernel: Y of one chunk from its entry state slot[n].
template <class C> __global__ __launch_bounds__(C::NT) void fwd_kernel(ChunkArgs a)
{
    typedef typename C::T T;
    constexpr int NFB = C::NFB, NEB = C::NEB, NTB = C::NTB, TT = C::TT;
    __shared__ FwdSmem<C> sm;
    const ChunkGeom G = chunk_geom<C>(a);
    const T *Q = (const T *)a.Q + G.hb, *K = (const T *)a.K + G.hb, *V = (const T *)a.V + G.hb;
    T *Y = (T *)a.out0 + G.hb;
    Frag<T> wf[NFB][NEB];
    if constexpr (C::FAVOR) load_wfrag<C>(wf, a.W);
    f4 rt[NFB][NEB];
    load_state_T<C>(rt, sm.Sl, slot_ptr<C>(a.slots, a, G.bh, G.nl));
    FwdRegs<C> rg;
    rg.load(Q, K, V, 0, G.len);
    for (int t0 = 0; t0 < G.len; t0 += TT) {
        const int nv = min(TT, G.len - t0);
        rg.store(sm, false);
        __syncthreads();
        if (t0 + TT < G.len) rg.load(Q, K, V, t0 + TT, G.len);
        f4 pq[NFB][NTB], pk[NTB][NFB];
        fwd_tile<C>(sm, wf, rt, nv, pq, pk);
        reduce_rows<C>(sm.red, nv, [&](int t, int e, f4 s, bool ok) {
            if (!ok) return;
            float dn = sm.redd[t];
#pragma unroll
            for (int w = 1; w < C::NW; ++w) dn += sm.redd[w * TT + t];
            store4<T>(Y + (size_t)(t0 + t) * C::D + e, s * (1.f / dn));
        });
        state_update_T<C>(sm, rt, pk);
        __syncthreads();
    }
}

}  // namespace slim
