// slim_kernels_bwd.h -- backward kernels of the chunked causal linear attention.
//
// Loss gradients follow from eq. (2) of the page "Sub-Linear Memory: How to Make
// Performers SLiM" (Subsection 2.1) by the chain rule.  Per row t of a chunk,
// with den_t the denominator and Y_t the output:
//   dNum_t = dY_t / den_t,          dden_t = -(dY_t . Y_t) / den_t,
//   A[t][s] = dNum_t . V_s + dden_t  for s <= t within the tile (else 0),
//   dg(Q_t) = sum_s A[t][s] g(K_s) + R_before dNum_t + dden_t S_before,
//   dg(K_s) = sum_t A[t][s] g(Q_t) + dR_after^T V_s + dS_after,
//   dV_s    = sum_t P[t][s] dNum_t + dR_after g(K_s),       P[t][s] = g(Q_t).g(K_s),
// where R_before is the state entering the tile, dR_after the gradient w.r.t. the
// state leaving it.  The state gradient is the backwards prefix sum of
// dNum_t g(Q_t)^T (and dden_t g(Q_t) for S), as Subsection 3.3 notes for PS.
// With the augmented value index (dNum's extra column = dden, V's = 1, R's = S,
// dR's = dS) every dden and dS term above is part of an MFMA.
// FAVOR+ chain: dq = sum_m dg_m g_m (w_m - q) (the -q sum vanishes for queries
// because Y_t is invariant under rescaling g(Q_t)); elu+1: dx = dg * g'(x).
#pragma once
#include "slim_kernels.h"

namespace slim {

// stats_kernel: recompute the chunk forward from slot[n] and write per row
// (1/den, dden) to stats.  dden = -(dY . Y) / den = -(dY . Num) / den^2 needs only
// two numbers per row from each wave -- its partial denominator and its partial
// dY . Num -- so the numerators themselves are never summed across waves.
template <class C> struct StatsSmem {
    FwdSmem<C, false> f;
    __align__(16) typename C::T xdy[C::XMat::SIZE];
};
template <class C>
__global__ __launch_bounds__(C::NT, waves_per_simd(sizeof(StatsSmem<C>), C::NW)) void stats_kernel(ChunkArgs a)
{
    typedef typename C::T T;
    constexpr int NFB = C::NFB, NEB = C::NEB, NEA = C::NEA, NTB = C::NTB, TT = C::TT, D = C::D, NW = C::NW;
    __shared__ StatsSmem<C> sm;
    const typename C::XMat xdy(sm.xdy);
    const ChunkGeom G = chunk_geom<C>(a);
    const int w = wave_id(), g = lgrp(), lc = lcol();
    const T *Q = (const T *)a.Q + G.hb, *K = (const T *)a.K + G.hb, *V = (const T *)a.V + G.hb;
    const T *dY = (const T *)a.dY + G.hb;
    float *st = a.stats + ((size_t)G.bh * a.P + G.nl) * (size_t)a.c * ROWSTAT;
    Frag<T> wf[NFB][NEB];
    if constexpr (C::FAVOR) load_wfrag<C>(wf, a.W);
    const float koff = key_off<C>(a);
    f4 rt[NFB][NEA];
    load_state_T<C>(rt, slot_ptr<C>(a.slots, a, G.bh, G.nl));
    FwdRegs<C> rg;
    typename C::Tile rdy;
    rg.load(Q, K, V, 0, G.len);
    rdy.load(dY, min(TT, G.len));
    for (int t0 = 0; t0 < G.len; t0 += TT) {
        const int nv = min(TT, G.len - t0);
        rg.store(sm.f, nv, koff);
        rdy.store(xdy, false, nullptr);
        __syncthreads();
        if (t0 + TT < G.len) {
            rg.load(Q, K, V, t0 + TT, G.len);
            rdy.load(dY + (size_t)(t0 + TT) * D, min(TT, G.len - t0 - TT));
        }
        f4 pq[NFB][NTB];
        float dot[NTB], den[NTB];
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) dot[tb] = den[tb] = 0.f;
        fwd_tile<C>(sm.f, wf, rt, pq, [&](int eb, int tb, f4 acc) {
            if (eb < NEB) {
                const f4 dy = xdy.get4(tb * 16 + lc, eb * 16 + 4 * g);
                dot[tb] += acc[0] * dy[0] + acc[1] * dy[1] + acc[2] * dy[2] + acc[3] * dy[3];
            } else {
                den[tb] = acc[0];  // row D of the numerators; zero in lanes with g > 0
            }
        });
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            float p = dot[tb];
            p += __shfl_xor(p, 16, 64);
            p += __shfl_xor(p, 32, 64);
            if (g == 0) {
                sm.f.red[((w * TT) + tb * 16 + lc) * 2] = den[tb];
                sm.f.red[((w * TT) + tb * 16 + lc) * 2 + 1] = p;
            }
        }
        __syncthreads();
        if (threadIdx.x < nv) {
            // the waves' partials rescaled to the common query offset, which the later
            // passes reuse
            const int t = threadIdx.x;
            float sc[NW], moff;
            wave_scales<C>(sm.f.qmax, t, sc, &moff);
            float dn = 0.f, dt = 0.f;
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                dn += sm.f.red[(v * TT + t) * 2] * sc[v];
                dt += sm.f.red[(v * TT + t) * 2 + 1] * sc[v];
            }
            const float inv = 1.f / dn;
            st[(size_t)(t0 + t) * ROWSTAT] = inv;
            st[(size_t)(t0 + t) * ROWSTAT + 1] = -dt * inv * inv;
            st[(size_t)(t0 + t) * ROWSTAT + 2] = moff;
            st[(size_t)(t0 + t) * ROWSTAT + 3] = 0.f;
        }
        state_update_T<C>(sm.f, rt);
        __syncthreads();
    }
}

// rowstat_kernel: the per-row statistics from what the forward kept: its output Y and,
// per row, 1/den at the common query offset and that offset (ChunkArgs::rstat); for the
// shapes whose dQ kernel does not make them itself (bwdq_makes_rowstats).
// dden = -(dY . Y) / den, since Y = Num / den; one row per VPR lanes (16-byte loads of
// Y and dY), the dot product reduced by lane shuffles.  Grid: (chunks of the window x
// parts of ROWSTAT_ROWS rows, heads), so that the launch has as many workgroups for
// long chunks as for short ones.
constexpr int ROWSTAT_NT = 256;
template <class C> __global__ __launch_bounds__(ROWSTAT_NT) void rowstat_kernel(ChunkArgs a)
{
    typedef typename C::T T;
    typedef typename Vec16<T>::type VT;
    constexpr int EPV = Vec16<T>::N, VPR = C::D / EPV, RPP = ROWSTAT_NT / VPR;
    static_assert(64 % VPR == 0, "a row's lanes stay in one wave");
    const int parts = (a.c + ROWSTAT_ROWS - 1) / ROWSTAT_ROWS;
    const int nl = blockIdx.x / parts, bh = blockIdx.y;
    const long long row0 = (long long)(a.n0 + nl) * a.c;
    const int len = (int)min((long long)a.c, a.L - row0);
    const int r0 = (blockIdx.x % parts) * ROWSTAT_ROWS, r1 = min(len, r0 + ROWSTAT_ROWS);
    const size_t hb = ((size_t)bh * (size_t)a.L + (size_t)row0) * C::D;
    const T *dY = (const T *)a.dY + hb, *Y = (const T *)a.Yin + hb;
    const float *rs = a.rstat + ((size_t)bh * a.L + row0) * 2;
    float *st = a.stats + ((size_t)bh * a.P + nl) * (size_t)a.c * ROWSTAT;
    const int sub = threadIdx.x % VPR, rsl = threadIdx.x / VPR;
    for (int t0 = r0; t0 < r1; t0 += RPP) {
        const int t = t0 + rsl;
        float p = 0.f;
        if (t < r1) {
            const VT y = gload<VT>(Y + (size_t)t * C::D + sub * EPV);
            const VT g = gload<VT>(dY + (size_t)t * C::D + sub * EPV);
#pragma unroll
            for (int j = 0; j < EPV; ++j) p = fmaf((float)y[j], (float)g[j], p);
        }
#pragma unroll
        for (int o = 1; o < VPR; o <<= 1) p += __shfl_xor(p, o, 64);
        if (t < r1 && sub == 0) {
            const float2 r = *reinterpret_cast<const float2 *>(rs + (size_t)t * 2);
            *reinterpret_cast<f4 *>(st + (size_t)t * ROWSTAT) = f4{r.x, -p * r.x, r.y, 0.f};
        }
    }
}

// gstate_kernel: gslot[n+1] = (dG_n, dGs_n) = sum over chunk n of
// (g(Q_t) dNum_t^T, dden_t g(Q_t)), the chunk's gradient w.r.t. its entry state
// (stored like a state slot), from Q, dY and the per-row statistics.
template <class C> struct GstateSmem {
    typedef typename C::T T;
    __align__(16) T xq[C::XMat::SIZE];
    __align__(16) T dn[C::XMat::SIZE];
    __align__(16) T dna[C::AuxMat::SIZE];
    __align__(16) T fq[C::NW * C::FMat::SIZE];
    float qoff[C::TT];
};
template <class C>
__global__ __launch_bounds__(C::NT, waves_per_simd(sizeof(GstateSmem<C>), C::NW)) void gstate_kernel(ChunkArgs a)
{
    typedef typename C::T T;
    constexpr int NFB = C::NFB, NEB = C::NEB, NEA = C::NEA, NTB = C::NTB, TT = C::TT, D = C::D;
    __shared__ GstateSmem<C> sm;
    const typename C::XMat xq(sm.xq);
    const AugTile<C> DN(sm.dn, sm.dna);
    const typename C::FMat Fq(sm.fq + wave_id() * C::FMat::SIZE);
    const ChunkGeom G = chunk_geom<C>(a);
    const T *Q = (const T *)a.Q + G.hb, *dY = (const T *)a.dY + G.hb;
    const float *st = a.stats + ((size_t)G.bh * a.P + G.nl) * (size_t)a.c * ROWSTAT;
    Frag<T> wf[NFB][NEB];
    if constexpr (C::FAVOR) load_wfrag<C>(wf, a.W);
    f4 dg[NFB][NEA];
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
        for (int eb = 0; eb < NEA; ++eb) dg[fb][eb] = f4zero();
    typename C::Tile rq, rdy;
    RowStatRegs<TT> rs;
    {
        const int n = min(TT, G.len);
        rq.load(Q, n);
        rdy.load(dY, n, st);
        rs.load(st, n);
    }
    for (int t0 = 0; t0 < G.len; t0 += TT) {
        rq.store(xq, false, nullptr);
        rdy.store(DN.x, true, nullptr);
        if (threadIdx.x < TT) {
            DN.set_aux(threadIdx.x, rs.dd);
            sm.qoff[threadIdx.x] = rs.qoff;
        }
        __syncthreads();
        if (t0 + TT < G.len) {
            const int n = min(TT, G.len - t0 - TT);
            rq.load(Q + (size_t)(t0 + TT) * D, n);
            rdy.load(dY + (size_t)(t0 + TT) * D, n, st + (size_t)(t0 + TT) * ROWSTAT);
            rs.load(st + (size_t)(t0 + TT) * ROWSTAT, n);
        }
        f4 pq[NFB][NTB];
        feat_T<C>(pq, xq, wf);
        q_finish_off<C>(pq, sm.qoff);
        put_features<C>(Fq, pq);
        wave_lds_fence();  // Fq written by this wave above
        // [dG | dGs] += g(Q)^T [dNum | dden] over this wave's features
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int eb = 0; eb < NEA; ++eb)
                mma_range<T>(dg[fb][eb], 0, NTB, [&](int tb) { return Fq.frag_r(fb * 16, tb * 16); },
                             [&](int tb) { return DN.fr(eb, tb * 16); });
        __syncthreads();
    }
    store_state_T<C>(slot_ptr<C>(a.gslots, a, G.bh, G.nl + 1), dg);
}

// State block with rows = value index e (incl. the auxiliary block, whose first
// row is the S / dS vector) and cols = this wave's features, from a slot.
template <class C> __device__ __forceinline__ void load_state_E(f4 (&r)[C::NEA][C::NFB], const float *slot)
{
    const int w = wave_id();
#pragma unroll
    for (int fb = 0; fb < C::NFB; ++fb) {
        const int m = w * C::MW + fb * 16 + lcol();
#pragma unroll
        for (int eb = 0; eb < C::NEB; ++eb)
#pragma unroll
            for (int j = 0; j < 4; ++j) r[eb][fb][j] = slot[(size_t)(eb * 16 + 4 * lgrp() + j) * C::M + m];
        r[C::NEB][fb] = f4{lgrp() == 0 ? slot[(size_t)C::D * C::M + m] : 0.f, 0.f, 0.f, 0.f};
    }
}

// Staging of the backward tiles: Q, K, V (+ ones), dNum = dY / den (+ dden).
template <class C> struct BwdRegs {
    typedef typename C::T T;
    typename C::Tile q, k, v, dy;
    RowStatRegs<C::TT> rs;
    // With the forward's output and its 8-byte row records (1/den', query offset): the
    // output tile and each vector's row offset, for the row statistics made here
    typename C::Tile y;
    float qo[C::Tile::PER];
    __device__ __forceinline__ void load(const T *Q, const T *K, const T *V, const T *dY, const float *st, int t0,
                                         int len)
    {
        const int n = min(C::TT, len - t0);
        q.load(Q + (size_t)t0 * C::D, n);
        k.load(K + (size_t)t0 * C::D, n);
        v.load(V + (size_t)t0 * C::D, n);
        dy.load(dY + (size_t)t0 * C::D, n, st + (size_t)t0 * ROWSTAT);
        rs.load(st + (size_t)t0 * ROWSTAT, n);
    }
    __device__ __forceinline__ void store(const typename C::XMat &xq, const typename C::XMat &xk,
                                          const AugTile<C> &Vt, const AugTile<C> &DN, float *kn2, float *qoff, int nv,
                                          float koff)
    {
        q.store(xq, false, nullptr);
        store_k_tile<C>(k, xk, kn2, nv, koff);
        store_v_tile<C>(v, Vt, nv);
        dy.store(DN.x, true, nullptr);
        if (threadIdx.x < C::TT) {
            DN.set_aux(threadIdx.x, rs.dd);
            qoff[threadIdx.x] = rs.qoff;
        }
    }
    // The same from the forward's output Y and row records fr ([row][2]: 1/den', offset):
    // each row's statistics (1/den, dden = -(dY . Y) / den, offset) are made here, put in
    // LDS for this tile and stored to st (the row-statistics layout) for the dK/dV pass.
    __device__ __forceinline__ void load_fwd(const T *Q, const T *K, const T *V, const T *dY, const float *fr,
                                             int t0, int len)
    {
        const int n = min(C::TT, len - t0);
        q.load(Q + (size_t)t0 * C::D, n);
        k.load(K + (size_t)t0 * C::D, n);
        v.load(V + (size_t)t0 * C::D, n);
        dy.load(dY + (size_t)t0 * C::D, n, fr + (size_t)t0 * 2, 2);
        const float *ob = uniform_ptr(fr + (size_t)t0 * 2);
#pragma unroll
        for (int i = 0; i < C::Tile::PER; ++i) {
            const int idx = threadIdx.x + i * C::NT, t = idx / C::Tile::VPR;
            qo[i] = idx < C::Tile::NV && t < n ? gload<float>(ob + (unsigned)(t * 2 + 1)) : 0.f;
        }
    }
    __device__ __forceinline__ void load_y(const T *Y, int t0, int len)
    {
        y.load(Y + (size_t)t0 * C::D, min(C::TT, len - t0));
    }
    __device__ __forceinline__ void store_fwd(const typename C::XMat &xq, const typename C::XMat &xk,
                                              const AugTile<C> &Vt, const AugTile<C> &DN, float *kn2, float *qoff,
                                              int nv, float koff, float *st)
    {
        constexpr int EPV = C::Tile::EPV, VPR = C::Tile::VPR;
        q.store(xq, false, nullptr);
        store_k_tile<C>(k, xk, kn2, nv, koff);
        store_v_tile<C>(v, Vt, nv);
        dy.store(DN.x, true, nullptr);
#pragma unroll
        for (int i = 0; i < C::Tile::PER; ++i) {
            const int idx = threadIdx.x + i * C::NT;
            const int t = idx / VPR, c = (idx % VPR) * EPV;
            float p = 0.f;  // dY . Y over the row: this lane's elements, then the row's lanes
#pragma unroll
            for (int j = 0; j < EPV; ++j) p = fmaf((float)y.v[i][j], (float)dy.v[i][j], p);
#pragma unroll
            for (int o = 1; o < VPR; o <<= 1) p += __shfl_xor(p, o, 64);
            if (idx < C::Tile::NV && c == 0) {
                const bool ok = t < nv;
                const float inv = dy.s[i], dd = ok ? -p * inv : 0.f;
                DN.set_aux(t, dd);
                qoff[t] = qo[i];
                if (ok) *reinterpret_cast<f4 *>(st + (size_t)t * ROWSTAT) = f4{inv, dd, qo[i], 0.f};
            }
        }
    }
};

// bwdq_kernel: dQ of one chunk.  Tiles in forward order, carrying the entry state
// [R; S] (rows e, cols m) from slot[n].  Where its registers allow (bf16 with d <= 32,
// or d = 64 with M >= 64; fp32 with d <= 32), it also accumulates the gstate_kernel's
// result from the g(Q) it already has, and the gstate_kernel is not launched.
// dQ's W^T product: with bf16 inputs, d <= 64 and a whole number of value blocks per
// wave count, the waves share dg(Q).g(Q) through LDS and each finishes whole output
// blocks from W^T fragments it holds (no partial sums); elsewhere (where the held
// fragments would cost spills) each wave reduces its own features' partial sums
// across waves through LDS.
// A wave owns value blocks w mod NEB + k NW (k < EBW): with fewer waves than value
// blocks it holds EBW x M/16 = NEB x NFB W^T fragments, as many as the partial-sum
// form does.
template <class C> struct DqShared {
    static constexpr bool value = C::FAVOR && sizeof(typename C::T) == 2 && C::D <= 64 &&
                                  (C::NW % C::NEB == 0 || C::NEB % C::NW == 0);
    static constexpr int EBW = C::NEB > C::NW ? C::NEB / C::NW : 1;
};
// W^T fragments of value block eb over all M features (free index e, contraction m),
// from the packed W^T.
template <class C>
__device__ __forceinline__ void load_wt_col(Frag<typename C::T> (&wt)[C::M / 16], const void *Wpv, int eb)
{
    typedef typename C::T T;
    const T *Wp = (const T *)Wpv;
#pragma unroll
    for (int mb = 0; mb < C::M / 16; ++mb)
        wt[mb] = *reinterpret_cast<const Frag<T> *>(Wp + (((size_t)eb * (C::M / 16) + mb) * 64 + threadIdx.x % 64) * 4);
}

// dW pass: one operand fragment of dg(X) . g(X) (four consecutive features m..m+3
// of tile row t) to the window's buffer; rows past the chunk's end are not stored.
template <class C>
__device__ __forceinline__ void store_pw(typename C::T *rows, int t, int nv, int m, Frag<typename C::T> v)
{
    bstore(rows, nv * C::M * (int)sizeof(typename C::T), (t * C::M + m) * (int)sizeof(typename C::T), v.v);
}
// The chunk's first row in a dW buffer (see ChunkArgs::pq).
template <class C> __device__ __forceinline__ typename C::T *pw_rows(void *buf, const ChunkArgs &a, const ChunkGeom &G)
{
    return (typename C::T *)buf + ((size_t)G.bh * a.P + G.nl) * (size_t)a.c * C::M;
}

// The dQ kernel makes the row statistics itself (from the forward's output and row
// records) where that costs it no spills: one vector of each input tile per thread
// (bf16), or fp32 (whose dQ kernel holds its registers at one wave per SIMD anyway).
// With two vectors per thread (two waves at d = 64, M = 64 before that shape moved to
// 16 features per wave) the extra tile spilled and the kernel went from 1.19 to 1.73 ms
// on 1M tokens x 8 heads, more than the separate pass costs (0.46 ms); at the 16K-token,
// 64-head shape the separate pass took 47 us and the dQ kernel gained 16.
// Features per wave of the dQ kernel.  At bf16, M = 64, 16 features per wave (four
// waves) instead of 32 (two) let it make the row statistics with no spill: on 1M tokens
// x 8 heads the dQ kernel went from 1.19 to 1.43 ms (it also reads Y now) and the 0.46 ms
// statistics pass went away.
template <typename T, int M> constexpr int bwdq_features_per_wave()
{
    return sizeof(T) == 2 && M == 64 ? 16 : 32;
}
template <class C> constexpr bool bwdq_makes_rowstats()
{
    return sizeof(typename C::T) == 4 || C::Tile::PER == 1;
}
// The dQ kernel also accumulates the gradient state from the g(Q) it has (instead of a
// separate pass over Q and dY) where its registers allow: at bf16, d = 128 with elu+1
// (no W fragments) it spills 40 B with the row statistics made in the kernel and still
// saves more than the pass costs (dQ + gstate 0.388 -> 0.368 ms at 8K tokens x 64
// heads, M = 128); FAVOR+ at d = 128 would spill 180-240 B.  At fp32 (one wave per
// SIMD, the accumulation registers in use) up to d = 64: 0.114 -> 0.097 ms at 4K tokens
// x 64 heads, M = 128; not at M = 256, where the g(Q) copy in LDS would leave 32-row
// tiles without room.
template <class C> constexpr bool bwdq_fuses_gstate()
{
    return C::D <= 32 || (sizeof(typename C::T) == 4 && C::D <= 64 && C::M >= 64 && C::M <= 128) ||
           (sizeof(typename C::T) == 2 && C::M >= 64 && (C::D <= 64 || (C::D <= 128 && !C::FAVOR)));
}
template <class C, bool FR = false> struct BwdqSmem {
    typedef typename C::T T;
    static constexpr bool DEFER_DQ = C::FAVOR && DqShared<C>::value && sizeof(T) == 2 && !FR;
    __align__(16) T xq[C::XMat::SIZE];
    __align__(16) T xk[C::XMat::SIZE];
    __align__(16) T xv[C::XMat::SIZE];
    __align__(16) T xva[C::AuxMat::SIZE];
    __align__(16) T dn[C::XMat::SIZE];
    __align__(16) T dna[C::AuxMat::SIZE];
    __align__(16) T fk[C::NW * C::FMat::SIZE];
    __align__(16) T fq[bwdq_fuses_gstate<C>() ? C::NW * C::FMat::SIZE : 8];
    // dg(Q) . g(Q) of the tile over all features (rows t, cols m), or the waves'
    // partial dQ sums (see DqShared)
    __align__(16) T gqm[DqShared<C>::value ? LMat<T, C::TT, C::M>::SIZE : 8];
    __align__(16) float red[C::FAVOR && !DqShared<C>::value ? C::NW * C::TT * C::LDR : 4];
    // the previous tile's dQ blocks as stored, each lane its own four values (bf16 shared
    // path without the row statistics made here)
    __align__(16) T dqs[DEFER_DQ ? ((C::TT / 16) * (C::D / 16) + C::NW - 1) / C::NW * C::NT * 4 : 8];
    float kn2[C::TT], qoff[C::TT];
};
// Waves per SIMD the dQ kernel is compiled for: three where 16 features per wave leave
// room for them (in registers and in LDS), else as the other chunk kernels.
template <class C> constexpr int bwdq_waves_per_simd()
{
    return C::MW == 16 && C::NW <= 4 && 3 * sizeof(BwdqSmem<C>) <= 160 * 1024 ? 3
                                                                                : waves_per_simd(sizeof(BwdqSmem<C>), C::NW);
}
// DW: also store dg(Q) . g(Q) for the projection gradient (slim_dw.h).  FR: the row
// statistics from the forward's output and row records (ChunkArgs::Yin, rstat), made
// per tile here and stored for the dK/dV pass; else read from ChunkArgs::stats.
template <class C, bool DW = false, bool FR = false>
__global__ __launch_bounds__(C::NT, bwdq_waves_per_simd<C>()) void bwdq_kernel(ChunkArgs a)
{
    typedef typename C::T T;
    constexpr int NFB = C::NFB, NEB = C::NEB, NEA = C::NEA, NTB = C::NTB, TT = C::TT, D = C::D, MW = C::MW;
    __shared__ BwdqSmem<C, FR> sm;
    float *red = sm.red, *kn2 = sm.kn2, *qoff = sm.qoff;
    const typename C::XMat xq(sm.xq), xk(sm.xk);
    const AugTile<C> Vt(sm.xv, sm.xva), DN(sm.dn, sm.dna);
    const typename C::FMat Fk(sm.fk + wave_id() * C::FMat::SIZE);
    const typename C::FMat Fq(sm.fq + wave_id() * C::FMat::SIZE);
    const ChunkGeom G = chunk_geom<C>(a);
    const int w = wave_id(), g = lgrp(), lc = lcol();
    const T *Q = (const T *)a.Q + G.hb, *K = (const T *)a.K + G.hb, *V = (const T *)a.V + G.hb;
    const T *dY = (const T *)a.dY + G.hb;
    T *dQ = (T *)a.out0 + G.hb;
    T *pw = DW ? pw_rows<C>(a.pq, a, G) : nullptr;
    constexpr bool FG = bwdq_fuses_gstate<C>();
    f4 dg[FG ? NFB : 1][FG ? NEA : 1];  // the chunk's gradient w.r.t. its entry state, own features
    if constexpr (FG)
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int eb = 0; eb < NEA; ++eb) dg[fb][eb] = f4zero();
    float *st = a.stats + ((size_t)G.bh * a.P + G.nl) * (size_t)a.c * ROWSTAT;
    const T *Yf = FR ? (const T *)a.Yin + G.hb : nullptr;
    const float *fr = FR ? a.rstat + ((size_t)G.bh * a.L + G.row0) * 2 : nullptr;
    Frag<T> wf[NFB][NEB];
    if constexpr (C::FAVOR) load_wfrag<C>(wf, a.W);
    const float koff = key_off<C>(a);
    f4 r[NEA][NFB];
    load_state_E<C>(r, slot_ptr<C>(a.slots, a, G.bh, G.nl));
    BwdRegs<C> rg;
    if constexpr (FR) {
        rg.load_fwd(Q, K, V, dY, fr, 0, G.len);
        rg.load_y(Yf, 0, G.len);
    } else {
        rg.load(Q, K, V, dY, st, 0, G.len);
    }
    // W^T fragments held over the tile loop (reloading them per tile put their cache
    // latency on the dQ chain).  Shared dg(Q).g(Q): a wave finishes the dQ^T blocks
    // (16 value columns x 16 rows) of value block w % NEB, over all features.
    // Otherwise: its own features, all value blocks.
    constexpr bool SH = DqShared<C>::value;
    constexpr int NB = NTB * NEB, MB = C::M / 16;
    const LMat<T, TT, C::M> Gq(sm.gqm);
    constexpr int EBW = DqShared<C>::EBW;
    Frag<T> wt[C::FAVOR ? (SH ? EBW * MB : NEB * NFB) : 1];
    if constexpr (C::FAVOR) {
        if constexpr (SH)
#pragma unroll
            for (int k = 0; k < EBW; ++k)
                load_wt_col<C>(*reinterpret_cast<Frag<T>(*)[MB]>(wt + k * MB), a.Wt, w % NEB + k * C::NW);
        else
#pragma unroll
            for (int eb = 0; eb < NEB; ++eb) load_wtfrag_block<C>(*reinterpret_cast<Frag<T>(*)[NFB]>(wt + eb * NFB), a.Wt, eb);
    }
    // dQ of a tile stored at the start of the next one (staged in LDS by each lane), so
    // that the wait for the next tile's inputs there does not also wait for these stores
    // to complete: the step that recomputes the row statistics 1.74 -> 1.70 ms at the
    // 16K-token, 64-head shape, the dW pass's dQ kernel 0.601 -> 0.592 ms.  Where the row
    // statistics are made here it spills (0.434 -> 0.449 ms).
    constexpr bool DEFER_DQ = BwdqSmem<C, FR>::DEFER_DQ;
    // Where several workgroups share a compute unit, the phases after the dQ exchange (the
    // W^T products, then the state updates) run at raised wave priority, as in the other
    // chunk kernels: 1.443 -> 1.424 ms on 1M tokens x 8 heads (M = 64, three workgroups per
    // CU).  Not for elu+1 (0.366 -> 0.371 ms at d = 128).
    constexpr bool PRIO_Q = C::FAVOR && SH && 4 * bwdq_waves_per_simd<C>() / C::NW >= 2;
    int pt0 = -1, pnv = 0;
    auto store_dq = [&]() {  // the values this lane staged in sm.dqs
#pragma unroll
        for (int j = 0; j < (NB + C::NW - 1) / C::NW; ++j) {
            const int blk = w + j * C::NW, tb = blk / NEB, eb = blk % NEB;
            if (blk >= NB) break;
            const int t = tb * 16 + lc;
            bstore(dQ + (size_t)pt0 * D, pnv * D * (int)sizeof(T), (t * D + eb * 16 + 4 * g) * (int)sizeof(T),
                   *reinterpret_cast<const bf4 *>(sm.dqs + ((size_t)j * C::NT + threadIdx.x) * 4));
        }
    };
    for (int t0 = 0; t0 < G.len; t0 += TT) {
        const int nv = min(TT, G.len - t0);
        if constexpr (FR)
            rg.store_fwd(xq, xk, Vt, DN, kn2, qoff, nv, koff, st + (size_t)t0 * ROWSTAT);
        else
            rg.store(xq, xk, Vt, DN, kn2, qoff, nv, koff);
        if constexpr (DEFER_DQ)
            if (pt0 >= 0) store_dq();
        __syncthreads();
        if constexpr (PRIO_Q) __builtin_amdgcn_s_setprio(0);
        if (t0 + TT < G.len) {
            if constexpr (FR) {
                rg.load_fwd(Q, K, V, dY, fr, t0 + TT, G.len);
                rg.load_y(Yf, t0 + TT, G.len);
            } else
                rg.load(Q, K, V, dY, st, t0 + TT, G.len);
        }
        f4 pq[NFB][NTB];
        feat_T<C>(pq, xq, wf);
        q_finish_off<C>(pq, qoff);
        if constexpr (FG) put_features<C>(Fq, pq);
        {
            f4 pkT[NFB][NTB];
            feat_T<C>(pkT, xk, wf);
            k_finish_T<C>(pkT, kn2);
            put_features<C>(Fk, pkT);
        }
        // A^T blocks (rows s, cols t), s <= t: [V | 1] [dNum | dden]^T
        Frag<T> at[NTB][NTB];  // 0 above the diagonal (s-block > t-block)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int sb = 0; sb < NTB; ++sb) {
                if (sb > tb) {
                    at[sb][tb] = cfrag<T>(f4zero());
                    continue;
                }
                f4 acc = f4zero();
                mma_range<T>(acc, 0, NEA, [&](int eb) { return Vt.fc(sb * 16, eb); },
                             [&](int eb) { return DN.fc(tb * 16, eb); });
                if (sb == tb)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (4 * g + j > lc) acc[j] = 0.f;
                at[sb][tb] = cfrag<T>(acc);
            }
        wave_lds_fence();  // Fk, Fq written by this wave above
        // dg(Q)^T blocks (rows m, cols t) = g(K)^T A^T + [R; S]^T [dNum | dden]^T
        f4 dq[NFB][NTB];
        // [R; S] += [V | 1]^T g(K), for the next tile (after its last use, in dq below).
        // Where the row statistics are made here and dg(Q).g(Q) is shared, issued before
        // the barrier of that exchange, so that these products overlap it: 0.437 -> 0.430
        // ms at the 16K-token, 64-head shape.  Without the statistics that spills; with 16
        // features per wave (three waves per SIMD) it was slower (1M tokens x 8 heads at
        // M = 64: 1.417 -> 1.444 ms).
        constexpr bool EARLY_R = FR && SH && C::FAVOR && MW >= 32;
        auto update_r = [&]() {
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
                for (int eb = 0; eb < NEA; ++eb)
                    mma_range<T>(r[eb][fb], 0, NTB, [&](int tb) { return Vt.fr(eb, tb * 16); },
                                 [&](int tb) { return Fk.frag_r(fb * 16, tb * 16); });
        };
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                f4 acc = f4zero();
                // (pairing these two lists, as the dK/dV kernel does, made this kernel spill:
                // 0.443 -> 0.508 ms at the 16K-token, 64-head shape)
                // over all s-blocks, the zero ones included (as in the forward)
                mma_range<T>(acc, 0, NTB, [&](int sb) { return Fk.frag_r(fb * 16, sb * 16); },
                             [&](int sb) { return at[sb][tb]; });
                mma_range<T>(acc, 0, NEA, [&](int eb) { return cfrag<T>(r[eb][fb]); },
                             [&](int eb) { return DN.fc(tb * 16, eb); });
                dq[fb][tb] = acc;
            }
        if constexpr (C::FAVOR) {
            // dQ^T (rows e, cols t) = W^T (dg(Q) . g(Q))^T
            if constexpr (SH) {
#pragma unroll
                for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
                    for (int tb = 0; tb < NTB; ++tb) {
                        const Frag<T> v = cfrag<T>(dq[fb][tb] * pq[fb][tb]);
                        Gq.put_frag(tb * 16 + lc, w * MW + fb * 16 + 4 * g, v);
                        if constexpr (DW) store_pw<C>(pw + (size_t)t0 * C::M, tb * 16 + lc, nv, w * MW + fb * 16 + 4 * g, v);
                    }
                if constexpr (EARLY_R) update_r();
                __syncthreads();
                if constexpr (PRIO_Q) __builtin_amdgcn_s_setprio(2);
#pragma unroll
                for (int j = 0; j < (NB + C::NW - 1) / C::NW; ++j) {
                    const int blk = w + j * C::NW, tb = blk / NEB, eb = blk % NEB;
                    if (blk >= NB) break;  // more waves than blocks
                    const int k = NEB > C::NW ? j % EBW : 0;  // eb = w mod NEB + k NW
                    f4 acc = f4zero();
                    mma_range<T>(acc, 0, MB, [&](int mb) { return wt[k * MB + mb]; },
                                 [&](int mb) { return Gq.frag_c(tb * 16, mb * 16); });
                    if constexpr (DEFER_DQ) {
                        *reinterpret_cast<bf4 *>(sm.dqs + ((size_t)j * C::NT + threadIdx.x) * 4) =
                            bf4{(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3]};
                    } else {
                        const int t = tb * 16 + lc;
                        bstore4<T>(dQ + (size_t)t0 * D, nv * D * (int)sizeof(T), (t * D + eb * 16 + 4 * g) * (int)sizeof(T), acc);
                    }
                }
                if constexpr (DEFER_DQ) {
                    pt0 = t0;
                    pnv = nv;
                }
            } else {
                Frag<T> gq[NFB][NTB];
#pragma unroll
                for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
                    for (int tb = 0; tb < NTB; ++tb) {
                        gq[fb][tb] = cfrag<T>(dq[fb][tb] * pq[fb][tb]);
                        if constexpr (DW)
                            store_pw<C>(pw + (size_t)t0 * C::M, tb * 16 + lc, nv, w * MW + fb * 16 + 4 * g, gq[fb][tb]);
                    }
#pragma unroll
                for (int eb = 0; eb < NEB; ++eb) {
#pragma unroll
                    for (int tb = 0; tb < NTB; ++tb) {
                        f4 acc = f4zero();
                        mma_range<T>(acc, 0, NFB, [&](int fb) { return wt[eb * NFB + fb]; },
                                     [&](int fb) { return gq[fb][tb]; });
                        put_red<C>(red, eb, tb, acc);
                    }
                }
                __syncthreads();
                reduce_rows<C>(red, nv, [&](int t, int e, f4 s, bool ok) {
                    bstore4<T>(dQ + (size_t)t0 * D, nv * D * (int)sizeof(T), (t * D + e) * (int)sizeof(T), s);
                });
            }
        } else {
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
                for (int tb = 0; tb < NTB; ++tb) {
                    const int t = tb * 16 + lc;
                    const f4 x = frag_to_f4<T>(xq.frag_c(tb * 16, w * MW + fb * 16));
                    f4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = dq[fb][tb][j] * elu1_grad(x[j]);
                    bstore4<T>(dQ + (size_t)t0 * D, nv * D * (int)sizeof(T), (t * D + w * MW + fb * 16 + 4 * g) * (int)sizeof(T), v);
                }
        }
        if constexpr (PRIO_Q) __builtin_amdgcn_s_setprio(1);
        if constexpr (!EARLY_R) update_r();
        // fused: [dG | dGs] += g(Q)^T [dNum | dden]
        if constexpr (FG)
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
                for (int eb = 0; eb < NEA; ++eb)
                    mma_range<T>(dg[fb][eb], 0, NTB, [&](int tb) { return Fq.frag_r(fb * 16, tb * 16); },
                                 [&](int tb) { return DN.fr(eb, tb * 16); });
        __syncthreads();
    }
    if constexpr (DEFER_DQ) store_dq();
    if constexpr (FG) store_state_T<C>(slot_ptr<C>(a.gslots, a, G.bh, G.nl + 1), dg);
}

// bwdkv_kernel: dK and dV of one chunk.  Tiles in reverse order, carrying the
// gradient w.r.t. the state after the tile, [dR; dS] (rows e, cols m), which
// starts from gslot[n+1].  The dV product also needs dR with the features as the
// contraction index: each tile a bf16 copy of this wave's dR block goes to the
// wave's own fp32 reduction rows (idle until the dV partials are written, which
// happens only after the last read of the copy) and is read back transposed; if
// it does not fit there, a second fp32 orientation is carried in registers.
template <class C> struct BwdkvSmem {
    typedef typename C::T T;
    typedef LMat<T, C::MW, C::D> DrMat;  // rows m, cols e
    static constexpr bool DR_IN_RED = DrMat::SIZE * sizeof(T) <= (size_t)C::TT * C::LDR * sizeof(float);
    __align__(16) float red[C::NW * C::TT * C::LDR];
    __align__(16) T xq[C::XMat::SIZE];
    __align__(16) T xk[C::XMat::SIZE];
    __align__(16) T xv[C::XMat::SIZE];
    __align__(16) T xva[C::AuxMat::SIZE];
    __align__(16) T dn[C::XMat::SIZE];
    __align__(16) T dna[C::AuxMat::SIZE];
    __align__(16) T fq[C::NW * C::FMat::SIZE];
    float kn2[C::TT], qoff[C::TT];
};
// dK's W^T product with shared operands: the waves put dg(K) . g(K) (bf16, all
// features) and their row-sum partials in the reduction rows, which are free once dV
// is stored, and each wave finishes whole dK blocks of the value blocks it owns from
// W^T fragments over all features, instead of reducing fp32 partial sums.  Used up to
// 64 features: there the fp32 reduction weighs most beside a tile's feature work (at
// d = 64, M = 64 the kernel goes from 1.91 to 1.67 ms on 1M tokens x 8 heads); at
// M = 256 the W^T fragments over all features cost more than the reduction saves
// (0.548 -> 0.60 ms at the 16K-token, 64-head shape).
template <class C> struct DkShared {
    typedef LMat<typename C::T, C::TT, C::M> GMat;
    static constexpr bool value = C::FAVOR && sizeof(typename C::T) == 2 && C::D <= 64 && C::M <= 64 &&
                                  GMat::SIZE * sizeof(typename C::T) + C::NW * C::TT * sizeof(float) <=
                                      (size_t)C::NW * C::TT * C::LDR * sizeof(float);
};
// DW: also store dg(K) . g(K) for the projection gradient (slim_dw.h).
template <class C, bool DW = false>
__global__ __launch_bounds__(C::NT, waves_per_simd(sizeof(BwdkvSmem<C>), C::NW)) void bwdkv_kernel(ChunkArgs a)
{
    typedef typename C::T T;
    constexpr int NFB = C::NFB, NEB = C::NEB, NEA = C::NEA, NTB = C::NTB, TT = C::TT, D = C::D, MW = C::MW;
    typedef typename BwdkvSmem<C>::DrMat DrMat;
    constexpr bool DRL = BwdkvSmem<C>::DR_IN_RED;
    __shared__ BwdkvSmem<C> sm;
    float *red = sm.red, *kn2 = sm.kn2, *qoff = sm.qoff;
    const typename C::XMat xq(sm.xq), xk(sm.xk);
    const AugTile<C> Vt(sm.xv, sm.xva), DN(sm.dn, sm.dna);
    const typename C::FMat Fq(sm.fq + wave_id() * C::FMat::SIZE);
    const DrMat Dr(reinterpret_cast<T *>(red + (size_t)wave_id() * TT * C::LDR));
    const ChunkGeom G = chunk_geom<C>(a);
    const int w = wave_id(), g = lgrp(), lc = lcol();
    const T *Q = (const T *)a.Q + G.hb, *K = (const T *)a.K + G.hb, *V = (const T *)a.V + G.hb;
    const T *dY = (const T *)a.dY + G.hb;
    T *dK = (T *)a.out1 + G.hb, *dV = (T *)a.out2 + G.hb;
    T *pw = DW ? pw_rows<C>(a.pk, a, G) : nullptr;
    const float *st = a.stats + ((size_t)G.bh * a.P + G.nl) * (size_t)a.c * ROWSTAT;
    const float *gsl = slot_ptr<C>(a.gslots, a, G.bh, G.nl + 1);
    const float koff = key_off<C>(a);
    f4 dr[NEA][NFB];                       // [dR; dS], rows e, cols m
    f4 drt[DRL ? 1 : NFB][DRL ? 1 : NEB];  // dR^T (rows m, cols e) when not copied through LDS
    load_state_E<C>(dr, gsl);
    if constexpr (!DRL) {
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int eb = 0; eb < NEB; ++eb)
                drt[fb][eb] = *reinterpret_cast<const f4 *>(gsl + (size_t)(eb * 16 + lc) * C::M + w * MW + fb * 16 +
                                                            4 * g);
    }

    const int last = ((G.len - 1) / TT) * TT;
    BwdRegs<C> rg;
    constexpr bool EARLY = C::Tile::PER == 1 && !DW;
    // dK of a tile, held in registers as stored, written during the next tile (after its
    // feature maps, whose waits for their W fragments would also wait for these stores):
    // where dK is made from each wave's own blocks (the shared-operand and elu+1 paths)
    // and a few registers hold it: 1.711 -> 1.613 ms on 1M tokens x 8 heads (M = 64),
    // 0.404 -> 0.400 ms for elu+1 at d = 128; the other path's values spill
    constexpr bool SHK = DkShared<C>::value;
    constexpr int EBW_ = NEB > C::NW ? NEB / C::NW : 1, TBS_ = C::NW > NEB ? C::NW / NEB : 1;
    constexpr int NDK_ = SHK ? EBW_ * NTB : NFB * NTB;
    constexpr bool DEFER_DK = !DW && (SHK || !C::FAVOR) && NDK_ <= 4;
    // Where dK is reduced across waves, the waves of a workgroup take raised issue priority
    // from dK's W^T products through both reductions (the phases that end a tile, paced by
    // LDS and memory latency), so that the other workgroup on the compute unit fills their
    // gaps rather than delaying them: 0.474 -> 0.444 ms at the 16K-token, 64-head shape
    // (the reductions alone 0.465, one level for all of it 0.444).  Not on the shared-operand
    // path, where it cost 1% on 1M tokens x 8 heads (M = 64), nor for elu+1 (no change).
    constexpr bool PRIO = C::FAVOR && !SHK;
    // On the shared-operand path with few features (W^T fragments of at most four feature
    // blocks for at most two value blocks per wave) the W and W^T fragments are loaded once
    // and held in registers over the tile loop instead of re-read every tile, where the
    // products right after the tile's barriers waited for them: on 1M tokens x 8 heads
    // (d = M = 64) 1.623 -> 1.525 ms for W^T, 1.48 ms with W too, still two waves per SIMD.
    // Not in the dW pass's variant, where they spill.
    constexpr int WR_EBW = NEB > C::NW ? NEB / C::NW : 1, WR_MB = C::M / 16;
    constexpr bool WT_REG = SHK && !DW && WR_MB <= 4 && WR_EBW <= 2;
    Frag<T> wtr[WT_REG ? WR_EBW : 1][WT_REG ? WR_MB : 1];
    Frag<T> wfr[WT_REG ? NFB : 1][WT_REG ? NEB : 1];
    if constexpr (WT_REG) {
        load_wfrag<C>(wfr, a.W);
#pragma unroll
        for (int k = 0; k < WR_EBW; ++k)
#pragma unroll
            for (int j = 0; j < WR_MB; ++j)
                wtr[k][j] = *reinterpret_cast<const Frag<T> *>((const T *)a.Wt +
                                                               (((size_t)(w % NEB + k * C::NW) * WR_MB + j) * 64 +
                                                                threadIdx.x % 64) * 4);
    }
    constexpr int NDK = DEFER_DK ? NDK_ : 1;
    typedef std::conditional_t<sizeof(T) == 2, bf4, f4> DkV;
    DkV dkv[NDK];
    int pt0 = -1, pnv = 0;
    auto pack = [](f4 x) -> DkV {
        if constexpr (sizeof(T) == 2)
            return DkV{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
        else
            return x;
    };
    auto store_dk = [&]() {
#pragma unroll
        for (int i = 0; i < NDK; ++i) {
            const int sb = i % NTB, s = sb * 16 + lc;
            int col;
            if constexpr (SHK) {
                if (sb % TBS_ != (w / NEB) % TBS_) continue;
                col = (w % NEB + (i / NTB) * C::NW) * 16 + 4 * g;
            } else {
                col = w * MW + (i / NTB) * 16 + 4 * g;
            }
            bstore(dK + (size_t)pt0 * D, pnv * D * (int)sizeof(T), (s * D + col) * (int)sizeof(T), dkv[i]);
        }
    };
    rg.load(Q, K, V, dY, st, last, G.len);
    for (int t0 = last; t0 >= 0; t0 -= TT) {
        const int nv = min(TT, G.len - t0);
        // W fragments, unless held (above), are re-read (from cache) every tile rather than
        // held over the loop; issued before the tile's staging and barrier, which cover their
        // latency
        Frag<T> wf[NFB][NEB];
        if constexpr (WT_REG) {
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
                for (int eb = 0; eb < NEB; ++eb) wf[fb][eb] = wfr[fb][eb];
        } else if constexpr (C::FAVOR)
            load_wfrag<C>(wf, a.W);
        rg.store(xq, xk, Vt, DN, kn2, qoff, nv, koff);
        __syncthreads();
        // the next tile's inputs: with one vector of each input tile per thread, in flight
        // over this whole tile (issued after the dK/dV products instead, their memory
        // latency showed: 0.521 -> 0.495 ms at the 16K-token, 64-head shape, 0.421 -> 0.401
        // for d = 128 elu+1); with two, the registers they hold cost more than that (1M
        // tokens at M = 64: 1.765 -> 1.810 ms), and in the dW pass's variant (0.706 ->
        // 0.718 ms); those fetch them during the gradient-state update
        if constexpr (EARLY)
            if (t0 > 0) rg.load(Q, K, V, dY, st, t0 - TT, G.len);
        Frag<T> fq[NFB][NTB], fkT[NFB][NTB];
        {
            f4 pq[NFB][NTB];
            feat_T<C>(pq, xq, wf);
            q_finish_off<C>(pq, qoff);
            to_frags<C>(fq, pq);
            put_feature_frags<C>(Fq, fq);
            f4 pkT[NFB][NTB];
            feat_T<C>(pkT, xk, wf);
            k_finish_T<C>(pkT, kn2);
            to_frags<C>(fkT, pkT);
        }
        if constexpr (DEFER_DK)
            if (pt0 >= 0) store_dk();
        if constexpr (DRL) {
#pragma unroll
            for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
                for (int fb = 0; fb < NFB; ++fb) Dr.put_frag(fb * 16 + lc, eb * 16 + 4 * g, cfrag<T>(dr[eb][fb]));
            // keep the compiler from holding these bf16 copies in registers until the dK
            // products below (it would otherwise reuse them there)
#pragma unroll
            for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
                for (int fb = 0; fb < NFB; ++fb) asm volatile("" : "+v"(dr[eb][fb]));
        }
        // dV^T blocks (rows e, cols s): dNum^T P + dR g(K)^T, reduced across waves.
        {
            Frag<T> fp[NTB][NTB];  // P[t][s] = g(Q_t).g(K_s) over own features; 0 for s > t
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int sb = 0; sb < NTB; ++sb) {
                    if (sb > tb) {
                        fp[tb][sb] = cfrag<T>(f4zero());
                        continue;
                    }
                    f4 acc = f4zero();
                    mma_range<T>(acc, 0, NFB, [&](int fb) { return fq[fb][tb]; }, [&](int fb) { return fkT[fb][sb]; });
                    if (sb == tb)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (lc > 4 * g + j) acc[j] = 0.f;
                    fp[tb][sb] = cfrag<T>(acc);
                }
            if constexpr (DRL) wave_lds_fence();  // Dr written by this wave above
            f4 dv[NEB][NTB];
#pragma unroll
            for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
                for (int sb = 0; sb < NTB; ++sb) {
                    // over all t-blocks, the zero ones included (one dNum operand pairing
                    // for every s-block, no zero-padded product)
                    f4 acc = f4zero();
                    mma_range<T>(acc, 0, NTB, [&](int tb) { return DN.fr(eb, tb * 16); },
                                 [&](int tb) { return fp[tb][sb]; });
                    if constexpr (DRL)
                        mma_range<T>(acc, 0, NFB, [&](int fb) { return Dr.frag_r(eb * 16, fb * 16); },
                                     [&](int fb) { return fkT[fb][sb]; });
                    else
                        mma_range<T>(acc, 0, NFB, [&](int fb) { return cfrag<T>(drt[fb][eb]); },
                                     [&](int fb) { return fkT[fb][sb]; });
                    dv[eb][sb] = acc;
                }
            // the partials overwrite this wave's dR copy: all its reads (of another type) first
            if constexpr (DRL) wave_lds_fence();
#pragma unroll
            for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
                for (int sb = 0; sb < NTB; ++sb) put_red<C>(red, eb, sb, dv[eb][sb]);
        }
        __syncthreads();
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(2);
        reduce_rows<C>(red, nv, [&](int s, int e, f4 v, bool ok) {
            bstore4<T>(dV + (size_t)t0 * D, nv * D * (int)sizeof(T), (s * D + e) * (int)sizeof(T), v);
        });
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
        __syncthreads();
        // dg(K)^T blocks (rows m, cols s) = g(Q)^T A + [dR; dS]^T [V | 1]^T,
        // A[t][s] = [dNum | dden]_t . [V | 1]_s for s <= t.
        f4 dk[NFB][NTB];
        {
            Frag<T> fa[NTB][NTB];
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int sb = 0; sb <= tb; ++sb) {
                    f4 acc = f4zero();
                    mma_range<T>(acc, 0, NEA, [&](int eb) { return DN.fc(tb * 16, eb); },
                                 [&](int eb) { return Vt.fc(sb * 16, eb); });
                    if (sb == tb)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (lc > 4 * g + j) acc[j] = 0.f;
                    fa[tb][sb] = cfrag<T>(acc);
                }
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
                for (int sb = 0; sb < NTB; ++sb) {
                    // the state list first, so that its blocks pair the same way for every
                    // sb (one set of operand registers for them)
                    f4 acc = f4zero();
                    mma_range2<T>(acc, 0, NEA, [&](int eb) { return cfrag<T>(dr[eb][fb]); },
                                  [&](int eb) { return Vt.fc(sb * 16, eb); }, sb, NTB,
                                  [&](int tb) { return Fq.frag_r(fb * 16, tb * 16); },
                                  [&](int tb) { return fa[tb][sb]; });
                    dk[fb][sb] = acc;
                }
        }
        // the gradient state (its last use, in the dg(K) products, is above): [dR; dS] +=
        // [dNum | dden]^T g(Q), for the tiles before (skipping it after the last tile took
        // the plain kernel from 0.564 to 0.541 ms; it slowed the dW pass's variant, which
        // keeps it)
        auto grad_state = [&]() {
#pragma unroll
            for (int fb = 0; fb < NFB && (DW || t0 > 0); ++fb) {
#pragma unroll
                for (int eb = 0; eb < NEA; ++eb)
                    mma_range<T>(dr[eb][fb], 0, NTB, [&](int tb) { return DN.fr(eb, tb * 16); },
                                 [&](int tb) { return Fq.frag_r(fb * 16, tb * 16); });
                if constexpr (!DRL) {
#pragma unroll
                    for (int eb = 0; eb < NEB; ++eb)
                        mma_range<T>(drt[fb][eb], 0, NTB, [&](int tb) { return Fq.frag_r(fb * 16, tb * 16); },
                                     [&](int tb) { return DN.fr(eb, tb * 16); });
                }
            }
        };
        // Issued before dK's W^T product and reduction rather than after them, so that these
        // matrix-core products overlap that work: at the 16K-token, 64-head shape 0.497 ->
        // 0.480 ms, on 1M tokens x 8 heads (M = 64) 1.708 -> 1.663 ms.  Not for the dW
        // pass's variant, whose extra stores fill that part (0.718 -> 0.752 ms there).
        if constexpr (!DW) {
            if constexpr (!EARLY)
                if (t0 > 0) rg.load(Q, K, V, dY, st, t0 - TT, G.len);
            grad_state();
        }
        if constexpr (DkShared<C>::value) {
            // dK = W^T-product of dg(K) . g(K) over all features - K * its row sum
            typedef typename DkShared<C>::GMat GMat;
            constexpr int MB = C::M / 16;
            const GMat Gk(reinterpret_cast<T *>(red));
            float *rsp = red + GMat::SIZE * sizeof(T) / sizeof(float);  // [NW][TT] row-sum partials
#pragma unroll
            for (int sb = 0; sb < NTB; ++sb) {
                Frag<T> gf[NFB];
#pragma unroll
                for (int fb = 0; fb < NFB; ++fb) {
                    gf[fb] = cfrag<T>(dk[fb][sb] * frag_to_f4<T>(fkT[fb][sb]));
                    Gk.put_frag(sb * 16 + lc, w * MW + fb * 16 + 4 * g, gf[fb]);
                    if constexpr (DW)
                        store_pw<C>(pw + (size_t)t0 * C::M, sb * 16 + lc, nv, w * MW + fb * 16 + 4 * g, gf[fb]);
                }
                // the row sums over the same rounded values that enter the W^T product (so
                // that W^T G - k sum(G) = sum_m G_m (w_m - k) cancels consistently for a key
                // close to a row of W), on the matrix cores: a row of ones times G
                f4 rs = f4zero();
                mma_range<T>(rs, 0, NFB, [&](int) { return ones_row0<T>(); }, [&](int fb) { return gf[fb]; });
                if (g == 0) rsp[w * TT + sb * 16 + lc] = rs[0];
            }
            // value blocks eb = w mod NW (all row blocks), or, with more waves than value
            // blocks, eb = w mod NEB and the row blocks sb = w / NEB mod NW / NEB
            constexpr int TB_STEP = C::NW > NEB ? C::NW / NEB : 1;
            constexpr int MH = MB >= 8 ? 8 : MB;  // W^T fragments held at once
            const T *Wp = (const T *)a.Wt;
            __syncthreads();
            constexpr int EBW = NEB > C::NW ? NEB / C::NW : 1;  // value blocks per wave
            auto dk_blocks = [&](int k) {
                const int eb = w % NEB + k * C::NW;
                f4 acc[NTB];
#pragma unroll
                for (int sb = 0; sb < NTB; ++sb) acc[sb] = f4zero();
#pragma unroll 1
                for (int m0 = 0; m0 < MB; m0 += MH) {
                    Frag<T> wt[MH];
#pragma unroll
                    for (int j = 0; j < MH; ++j) {
                        if constexpr (WT_REG)
                            wt[j] = wtr[k][m0 + j];
                        else
                            wt[j] = *reinterpret_cast<const Frag<T> *>(
                                Wp + (((size_t)eb * MB + m0 + j) * 64 + threadIdx.x % 64) * 4);
                    }
#pragma unroll
                    for (int sb = 0; sb < NTB; ++sb) {
                        if (sb % TB_STEP != (w / NEB) % TB_STEP) continue;
                        mma_range<T>(acc[sb], 0, MH, [&](int mb) { return wt[mb]; },
                                     [&](int mb) { return Gk.frag_c(sb * 16, (m0 + mb) * 16); });
                    }
                }
#pragma unroll
                for (int sb = 0; sb < NTB; ++sb) {
                    if (sb % TB_STEP != (w / NEB) % TB_STEP) continue;
                    const int s = sb * 16 + lc;
                    float rs = rsp[s];
#pragma unroll
                    for (int w2 = 1; w2 < C::NW; ++w2) rs += rsp[w2 * TT + s];
                    const f4 r = acc[sb] - xk.get4(s, eb * 16 + 4 * g) * rs;
                    if constexpr (DEFER_DK)
                        dkv[k * NTB + sb] = pack(r);
                    else
                        bstore4<T>(dK + (size_t)t0 * D, nv * D * (int)sizeof(T), (s * D + eb * 16 + 4 * g) * (int)sizeof(T), r);
                }
            };
            if constexpr (DEFER_DK) {
#pragma unroll
                for (int k = 0; k < EBW; ++k) dk_blocks(k);
            } else {
#pragma unroll 1
                for (int k = 0; k < EBW; ++k) dk_blocks(k);
            }
        } else if constexpr (C::FAVOR) {
            // dK^T = W^T (dg(K) . g(K))^T and the row sums of dg(K) . g(K), reduced across
            // waves (the sums in column D of the reduction rows); dK = that - K * rowsum.
            Frag<T> gk[NFB][NTB];
#pragma unroll
            for (int sb = 0; sb < NTB; ++sb) {
#pragma unroll
                for (int fb = 0; fb < NFB; ++fb) {
                    gk[fb][sb] = cfrag<T>(dk[fb][sb] * frag_to_f4<T>(fkT[fb][sb]));
                    if constexpr (DW)
                        store_pw<C>(pw + (size_t)t0 * C::M, sb * 16 + lc, nv, w * MW + fb * 16 + 4 * g, gk[fb][sb]);
                }
                // row sums of the values as rounded for the W^T product, on the matrix
                // cores: a row of ones times dg(K) . g(K)
                f4 rs = f4zero();
                mma_range<T>(rs, 0, NFB, [&](int) { return ones_row0<T>(); }, [&](int fb) { return gk[fb][sb]; });
                if (g == 0) red[(w * TT + sb * 16 + lc) * C::LDR + D] = rs[0];
            }
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
            auto wt_block = [&](int eb) {
                Frag<T> wt[NFB];
                load_wtfrag_block<C>(wt, a.Wt, eb);
#pragma unroll
                for (int sb = 0; sb < NTB; ++sb) {
                    f4 acc = f4zero();
                    mma_range<T>(acc, 0, NFB, [&](int fb) { return wt[fb]; }, [&](int fb) { return gk[fb][sb]; });
                    put_red<C>(red, eb, sb, acc);
                }
            };
            // W^T blocks two at a time (their loads issued together): 0.449 -> 0.436 ms at the
            // 16K-token, 64-head shape, fp32 at d = 64, M = 128 0.1065 -> 0.1052 ms; all four at
            // once spill there.  One at a time in the dW pass's variant (0.659 -> 0.665 ms).
            if constexpr (DW) {
#pragma unroll 1
                for (int eb = 0; eb < NEB; ++eb) wt_block(eb);
            } else {
#pragma unroll 2
                for (int eb = 0; eb < NEB; ++eb) wt_block(eb);
            }
            __syncthreads();
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(2);
            reduce_rows<C>(red, nv, [&](int s, int e, f4 v, bool ok) {
                bstore4<T>(dK + (size_t)t0 * D, nv * D * (int)sizeof(T), (s * D + e) * (int)sizeof(T),
                           v - xk.get4(s, e) * reduce_col<C>(red, s));
            });
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
        } else {
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
                for (int sb = 0; sb < NTB; ++sb) {
                    const int s = sb * 16 + lc;
                    const f4 x = frag_to_f4<T>(xk.frag_c(sb * 16, w * MW + fb * 16));
                    f4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = dk[fb][sb][j] * elu1_grad(x[j]);
                    if constexpr (DEFER_DK)
                        dkv[fb * NTB + sb] = pack(v);
                    else
                        bstore4<T>(dK + (size_t)t0 * D, nv * D * (int)sizeof(T), (s * D + w * MW + fb * 16 + 4 * g) * (int)sizeof(T), v);
                }
        }
        if constexpr (DW) {
            if (t0 > 0) rg.load(Q, K, V, dY, st, t0 - TT, G.len);
            grad_state();
        }
        if constexpr (DEFER_DK) {
            pt0 = t0;
            pnv = nv;
        }
        __syncthreads();
    }
    if constexpr (DEFER_DK) store_dk();
}

}  // namespace slim
