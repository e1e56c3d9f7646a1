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
// FAVOR+ chain: dq = sum_m dg_m g_m (w_m - q) (the -q sum vanishes for queries
// because Y_t is invariant under rescaling g(Q_t)); elu+1: dx = dg * g'(x).
#pragma once
#include "slim_kernels.h"

namespace slim {

// stats_kernel: recompute the chunk forward from slot[n]; write per-row
// (1/den, dden) to stats and gslot[n+1] = (dG_n, dGs_n) = sum over the chunk of
// (dNum_t g(Q_t)^T, dden_t g(Q_t)) -- the chunk's gradient w.r.t. its entry state.
template <class C> __global__ __launch_bounds__(C::NT) void stats_kernel(ChunkArgs a)
{
    typedef typename C::T T;
    constexpr int NFB = C::NFB, NEB = C::NEB, NTB = C::NTB, TT = C::TT, D = C::D;
    __shared__ FwdSmem<C> sm;
    __shared__ __align__(16) T xdy[TT * C::LDX];
    __shared__ __align__(16) T dnt[D * C::LDT];
    __shared__ float ddl[TT];
    const ChunkGeom G = chunk_geom<C>(a);
    const int w = wave_id(), g = lgrp(), lc = lcol();
    const T *Q = (const T *)a.Q + G.hb, *K = (const T *)a.K + G.hb, *V = (const T *)a.V + G.hb;
    const T *dY = (const T *)a.dY + G.hb;
    float *st = a.stats + ((size_t)G.bh * a.P + G.nl) * (size_t)a.c * 2;
    Frag<T> wf[NFB][NEB];
    if constexpr (C::FAVOR) load_wfrag<C>(wf, a.W);
    f4 rt[NFB][NEB], dg[NFB][NEB];
    float gs[NFB];
    load_state_T<C>(rt, sm.Sl, slot_ptr<C>(a.slots, a, G.bh, G.nl));
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) {
        gs[fb] = 0.f;
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb) dg[fb][eb] = f4zero();
    }
    FwdRegs<C> rg;
    typename C::Tile rdy;
    rg.load(Q, K, V, 0, G.len);
    rdy.load(dY, min(TT, G.len));
    for (int t0 = 0; t0 < G.len; t0 += TT) {
        const int nv = min(TT, G.len - t0);
        rg.store(sm, true);
        rdy.store(xdy, C::LDX, nullptr, 0, false, nullptr);
        __syncthreads();
        if (t0 + TT < G.len) {
            rg.load(Q, K, V, t0 + TT, G.len);
            rdy.load(dY + (size_t)(t0 + TT) * D, min(TT, G.len - t0 - TT));
        }
        f4 pq[NFB][NTB], pk[NTB][NFB];
        fwd_tile<C>(sm, wf, rt, nv, pq, pk);
        reduce_rows<C>(sm.red, nv, [&](int t, int e, f4 s, bool ok) {
            float dn = sm.redd[t];
#pragma unroll
            for (int ww = 1; ww < C::NW; ++ww) dn += sm.redd[ww * TT + t];
            const float inv = ok ? 1.f / dn : 0.f;
            const f4 y = s * inv;
            const f4 dy = load4<T>(xdy + t * C::LDX + e);
            float p = dy[0] * y[0] + dy[1] * y[1] + dy[2] * y[2] + dy[3] * y[3];
#pragma unroll
            for (int o = 1; o < D / 4; o <<= 1) p += __shfl_xor(p, o, 64);
#pragma unroll
            for (int j = 0; j < 4; ++j) dnt[(e + j) * C::LDT + t] = (T)(dy[j] * inv);
            if (e == 0) {
                const float dd = ok ? -p * inv : 0.f;
                ddl[t] = dd;
                if (ok) {
                    st[(size_t)(t0 + t) * 2] = inv;
                    st[(size_t)(t0 + t) * 2 + 1] = dd;
                }
            }
        });
        __syncthreads();
        f4 pqS[NTB][NFB];
        feat_S<C>(pqS, sm.xq, sm.qt, wf);
        q_finish_S<C>(pqS, sm.qmax);
        Frag<T> fqS[NTB][NFB];
        to_frags<C>(fqS, pqS);
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb) {
#pragma unroll
            for (int eb = 0; eb < NEB; ++eb)
                mma_range<T>(dg[fb][eb], 0, NTB, [&](int tb) { return fqS[tb][fb]; },
                             [&](int tb) { return lds_frag<T>(dnt, C::LDT, eb * 16, tb * 16); });
            float s = 0.f;
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int j = 0; j < 4; ++j) s += pqS[tb][fb][j] * ddl[tb * 16 + 4 * g + j];
            gs[fb] += sum_groups(s);
        }
        state_update_T<C>(sm, rt, pk);
        __syncthreads();
    }
    float *out = slot_ptr<C>(a.gslots, a, G.bh, G.nl + 1);
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) {
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb)
            *reinterpret_cast<f4 *>(out + (size_t)(eb * 16 + lc) * C::M + w * C::MW + fb * 16 + 4 * g) = dg[fb][eb];
        if (g == 0) out[D * C::M + w * C::MW + fb * 16 + lc] = gs[fb];
    }
}

// bwdq_kernel: dQ of one chunk.  Tiles in forward order, carrying the entry
// state R (blocks with rows e, cols m) and S from slot[n].
template <class C> __global__ __launch_bounds__(C::NT) void bwdq_kernel(ChunkArgs a)
{
    typedef typename C::T T;
    constexpr int NFB = C::NFB, NEB = C::NEB, NTB = C::NTB, TT = C::TT, D = C::D, M = C::M, MW = C::MW;
    __shared__ __align__(16) T xq[TT * C::LDX];
    __shared__ __align__(16) T xk[TT * C::LDX];
    __shared__ __align__(16) T kt[C::FAVOR ? 8 : D * C::LDT];
    __shared__ __align__(16) T xv[TT * C::LDX];
    __shared__ __align__(16) T vt[D * C::LDT];
    __shared__ __align__(16) T dn[TT * C::LDX];
    __shared__ __align__(16) float red[C::FAVOR ? C::NW * TT * C::LDR : 4];
    __shared__ float invl[TT], ddl[TT], kn[TT], qmax[C::NW * TT], Sl[M];
    const ChunkGeom G = chunk_geom<C>(a);
    const int w = wave_id(), g = lgrp(), lc = lcol();
    const T *Q = (const T *)a.Q + G.hb, *K = (const T *)a.K + G.hb, *V = (const T *)a.V + G.hb;
    const T *dY = (const T *)a.dY + G.hb;
    T *dQ = (T *)a.out0 + G.hb;
    const float *st = a.stats + ((size_t)G.bh * a.P + G.nl) * (size_t)a.c * 2;
    Frag<T> wf[NFB][NEB], wt[NEB][NFB];
    if constexpr (C::FAVOR) {
        load_wfrag<C>(wf, a.W);
        load_wtfrag<C>(wt, a.W);
    }
    const float *slot = slot_ptr<C>(a.slots, a, G.bh, G.nl);
    f4 r[NEB][NFB];  // R: rows e, cols m
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int j = 0; j < 4; ++j) r[eb][fb][j] = slot[(size_t)(eb * 16 + 4 * g + j) * M + w * MW + fb * 16 + lc];
    for (int m = threadIdx.x; m < M; m += C::NT) Sl[m] = slot[D * M + m];

    typename C::Tile rq, rk, rv, rdy;
    RowStatRegs<TT> rs;
    auto prefetch = [&](int t) {
        const int n = min(TT, G.len - t);
        rq.load(Q + (size_t)t * D, n);
        rk.load(K + (size_t)t * D, n);
        rv.load(V + (size_t)t * D, n);
        rdy.load(dY + (size_t)t * D, n, st + (size_t)t * 2);
        rs.load(st + (size_t)t * 2, n);
    };
    prefetch(0);
    for (int t0 = 0; t0 < G.len; t0 += TT) {
        const int nv = min(TT, G.len - t0);
        rq.store(xq, C::LDX, nullptr, 0, false, nullptr);
        rk.store(xk, C::LDX, C::FAVOR ? nullptr : kt, C::LDT, false, C::FAVOR ? kn : nullptr);
        rv.store(xv, C::LDX, vt, C::LDT, false, nullptr);
        rdy.store(dn, C::LDX, nullptr, 0, true, nullptr);
        rs.store(invl, ddl);
        __syncthreads();
        if (t0 + TT < G.len) prefetch(t0 + TT);
        f4 pq[NFB][NTB], pk[NTB][NFB];
        feat_T<C>(pq, xq, wf);
        if constexpr (C::FAVOR) q_partial_max<C>(pq, qmax);
        __syncthreads();
        q_finish_T<C>(pq, qmax);
        feat_S<C>(pk, xk, kt, wf);
        k_finish_S<C>(pk, kn, nv);
        // A^T blocks (rows s, cols t), s <= t
        f4 at[NTB][NTB];
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int sb = 0; sb <= tb; ++sb) {
                f4 acc = f4zero();
                mma_range<T>(acc, 0, NEB, [&](int kb) { return lds_frag<T>(xv, C::LDX, sb * 16, kb * 16); },
                             [&](int kb) { return lds_frag<T>(dn, C::LDX, tb * 16, kb * 16); });
                const float dd = ddl[tb * 16 + lc];
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = (sb == tb && 4 * g + j > lc) ? 0.f : acc[j] + dd;
                at[sb][tb] = acc;
            }
        // dg(Q)^T blocks (rows m, cols t)
        f4 dq[NFB][NTB];
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                f4 acc = f4zero();
                mma_range<T>(acc, 0, tb + 1, [&](int sb) { return cfrag<T>(pk[sb][fb]); },
                             [&](int sb) { return cfrag<T>(at[sb][tb]); });
                mma_range<T>(acc, 0, NEB, [&](int eb) { return cfrag<T>(r[eb][fb]); },
                             [&](int eb) { return lds_frag<T>(dn, C::LDX, tb * 16, eb * 16); });
                const float dd = ddl[tb * 16 + lc];
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] += Sl[w * MW + fb * 16 + 4 * g + j] * dd;
                dq[fb][tb] = acc;
            }
        if constexpr (C::FAVOR) {
            // dQ^T (rows e, cols t) = W^T (dg(Q) . g(Q))^T over own features, reduced across waves
            Frag<T> gq[NFB][NTB];
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
                for (int tb = 0; tb < NTB; ++tb) gq[fb][tb] = cfrag<T>(dq[fb][tb] * pq[fb][tb]);
#pragma unroll
            for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
                for (int tb = 0; tb < NTB; ++tb) {
                    f4 acc = f4zero();
                    mma_range<T>(acc, 0, NFB, [&](int fb) { return wt[eb][fb]; }, [&](int fb) { return gq[fb][tb]; });
                    *reinterpret_cast<f4 *>(red + (w * TT + tb * 16 + lc) * C::LDR + eb * 16 + 4 * g) = acc;
                }
            __syncthreads();
            reduce_rows<C>(red, nv, [&](int t, int e, f4 s, bool ok) {
                if (ok) store4<T>(dQ + (size_t)(t0 + t) * D + e, s);
            });
        } else {
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
                for (int tb = 0; tb < NTB; ++tb) {
                    const int t = tb * 16 + lc;
                    const f4 x = frag_to_f4<T>(lds_frag<T>(xq, C::LDX, tb * 16, w * MW + fb * 16));
                    f4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = dq[fb][tb][j] * elu1_grad(x[j]);
                    if (t < nv) store4<T>(dQ + (size_t)(t0 + t) * D + w * MW + fb * 16 + 4 * g, v);
                }
        }
        // R += V^T g(K), S += sum g(K)
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb) {
#pragma unroll
            for (int eb = 0; eb < NEB; ++eb)
                mma_range<T>(r[eb][fb], 0, NTB, [&](int tb) { return lds_frag<T>(vt, C::LDT, eb * 16, tb * 16); },
                             [&](int tb) { return cfrag<T>(pk[tb][fb]); });
            float s = 0.f;
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) s += pk[tb][fb][0] + pk[tb][fb][1] + pk[tb][fb][2] + pk[tb][fb][3];
            s = sum_groups(s);
            if (g == 0) Sl[w * MW + fb * 16 + lc] += s;
        }
        __syncthreads();
    }
}

// bwdkv_kernel: dK and dV of one chunk.  Tiles in reverse order, carrying the
// gradient w.r.t. the state after the tile (dR in both orientations, dS), which
// starts from gslot[n+1].
template <class C> __global__ __launch_bounds__(C::NT) void bwdkv_kernel(ChunkArgs a)
{
    typedef typename C::T T;
    constexpr int NFB = C::NFB, NEB = C::NEB, NTB = C::NTB, TT = C::TT, D = C::D, M = C::M, MW = C::MW;
    __shared__ __align__(16) T xq[TT * C::LDX];
    __shared__ __align__(16) T qt[C::FAVOR ? 8 : D * C::LDT];
    __shared__ __align__(16) T xk[TT * C::LDX];
    __shared__ __align__(16) T xv[TT * C::LDX];
    __shared__ __align__(16) T dn[TT * C::LDX];
    __shared__ __align__(16) T dnt[D * C::LDT];
    __shared__ __align__(16) float red[C::NW * TT * C::LDR];
    __shared__ float redk[C::NW * TT];
    __shared__ float invl[TT], ddl[TT], kn[TT], qmax[C::NW * TT], dSl[M];
    const ChunkGeom G = chunk_geom<C>(a);
    const int w = wave_id(), g = lgrp(), lc = lcol();
    const T *Q = (const T *)a.Q + G.hb, *K = (const T *)a.K + G.hb, *V = (const T *)a.V + G.hb;
    const T *dY = (const T *)a.dY + G.hb;
    T *dK = (T *)a.out1 + G.hb, *dV = (T *)a.out2 + G.hb;
    const float *st = a.stats + ((size_t)G.bh * a.P + G.nl) * (size_t)a.c * 2;
    Frag<T> wf[NFB][NEB], wt[NEB][NFB];
    if constexpr (C::FAVOR) {
        load_wfrag<C>(wf, a.W);
        load_wtfrag<C>(wt, a.W);
    }
    const float *gsl = slot_ptr<C>(a.gslots, a, G.bh, G.nl + 1);
    f4 dr[NEB][NFB], drt[NFB][NEB];
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb) {
#pragma unroll
            for (int j = 0; j < 4; ++j) dr[eb][fb][j] = gsl[(size_t)(eb * 16 + 4 * g + j) * M + w * MW + fb * 16 + lc];
            drt[fb][eb] = *reinterpret_cast<const f4 *>(gsl + (size_t)(eb * 16 + lc) * M + w * MW + fb * 16 + 4 * g);
        }
    for (int m = threadIdx.x; m < M; m += C::NT) dSl[m] = gsl[D * M + m];

    const int last = ((G.len - 1) / TT) * TT;
    typename C::Tile rq, rk, rv, rdy;
    RowStatRegs<TT> rs;
    auto prefetch = [&](int t) {
        const int n = min(TT, G.len - t);
        rq.load(Q + (size_t)t * D, n);
        rk.load(K + (size_t)t * D, n);
        rv.load(V + (size_t)t * D, n);
        rdy.load(dY + (size_t)t * D, n, st + (size_t)t * 2);
        rs.load(st + (size_t)t * 2, n);
    };
    prefetch(last);
    for (int t0 = last; t0 >= 0; t0 -= TT) {
        const int nv = min(TT, G.len - t0);
        rq.store(xq, C::LDX, C::FAVOR ? nullptr : qt, C::LDT, false, nullptr);
        rk.store(xk, C::LDX, nullptr, 0, false, C::FAVOR ? kn : nullptr);
        rv.store(xv, C::LDX, nullptr, 0, false, nullptr);
        rdy.store(dn, C::LDX, dnt, C::LDT, true, nullptr);
        rs.store(invl, ddl);
        __syncthreads();
        if (t0 > 0) prefetch(t0 - TT);
        // Features, kept as MFMA operand fragments (the fp32 blocks die at once).
        Frag<T> fq[NFB][NTB], fqS[NTB][NFB], fkT[NFB][NTB];
        {
            f4 pq[NFB][NTB];
            feat_T<C>(pq, xq, wf);
            if constexpr (C::FAVOR) q_partial_max<C>(pq, qmax);
            __syncthreads();
            q_finish_T<C>(pq, qmax);
            to_frags<C>(fq, pq);
        }
        {
            f4 pqS[NTB][NFB];
            feat_S<C>(pqS, xq, qt, wf);
            q_finish_S<C>(pqS, qmax);
            to_frags<C>(fqS, pqS);
        }
        {
            f4 pkT[NFB][NTB];
            feat_T<C>(pkT, xk, wf);
            k_finish_T<C>(pkT, kn, nv);
            to_frags<C>(fkT, pkT);
        }
        // dV^T blocks (rows e, cols s): dNum^T P + dR g(K)^T, reduced across waves.
        // P[t][s] = g(Q_t).g(K_s) over this wave's features, s <= t.
        {
            Frag<T> fp[NTB][NTB];
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int sb = 0; sb <= tb; ++sb) {
                    f4 acc = f4zero();
                    mma_range<T>(acc, 0, NFB, [&](int fb) { return fq[fb][tb]; }, [&](int fb) { return fkT[fb][sb]; });
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (sb == tb && lc > 4 * g + j) acc[j] = 0.f;
                    fp[tb][sb] = cfrag<T>(acc);
                }
#pragma unroll
            for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
                for (int sb = 0; sb < NTB; ++sb) {
                    f4 acc = f4zero();
                    mma_range<T>(acc, sb, NTB, [&](int tb) { return lds_frag<T>(dnt, C::LDT, eb * 16, tb * 16); },
                                 [&](int tb) { return fp[tb][sb]; });
                    mma_range<T>(acc, 0, NFB, [&](int fb) { return cfrag<T>(drt[fb][eb]); },
                                 [&](int fb) { return fkT[fb][sb]; });
                    *reinterpret_cast<f4 *>(red + (w * TT + sb * 16 + lc) * C::LDR + eb * 16 + 4 * g) = acc;
                }
        }
        __syncthreads();
        reduce_rows<C>(red, nv, [&](int s, int e, f4 v, bool ok) {
            if (ok) store4<T>(dV + (size_t)(t0 + s) * D + e, v);
        });
        __syncthreads();
        // dg(K)^T blocks (rows m, cols s): A^T g(Q) + dR^T V + dS, with
        // A[t][s] = dNum_t . V_s + dden_t for s <= t (the full sum over d, every wave).
        f4 dk[NFB][NTB];
        {
            Frag<T> fa[NTB][NTB];
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int sb = 0; sb <= tb; ++sb) {
                    f4 acc = f4zero();
                    mma_range<T>(acc, 0, NEB, [&](int kb) { return lds_frag<T>(dn, C::LDX, tb * 16, kb * 16); },
                                 [&](int kb) { return lds_frag<T>(xv, C::LDX, sb * 16, kb * 16); });
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[j] = (sb == tb && lc > 4 * g + j) ? 0.f : acc[j] + ddl[tb * 16 + 4 * g + j];
                    fa[tb][sb] = cfrag<T>(acc);
                }
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
                for (int sb = 0; sb < NTB; ++sb) {
                    f4 acc = f4zero();
                    mma_range<T>(acc, sb, NTB, [&](int tb) { return fqS[tb][fb]; }, [&](int tb) { return fa[tb][sb]; });
                    mma_range<T>(acc, 0, NEB, [&](int eb) { return cfrag<T>(dr[eb][fb]); },
                                 [&](int eb) { return lds_frag<T>(xv, C::LDX, sb * 16, eb * 16); });
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[j] += dSl[w * MW + fb * 16 + 4 * g + j];
                    dk[fb][sb] = acc;
                }
        }
        if constexpr (C::FAVOR) {
            // dK = (dg(K) . g(K)) W - K * rowsum(dg(K) . g(K)), reduced across waves
            Frag<T> gk[NFB][NTB];
#pragma unroll
            for (int sb = 0; sb < NTB; ++sb) {
                float rsum = 0.f;
#pragma unroll
                for (int fb = 0; fb < NFB; ++fb) {
                    const f4 gg = dk[fb][sb] * frag_to_f4<T>(fkT[fb][sb]);
                    rsum += gg[0] + gg[1] + gg[2] + gg[3];
                    gk[fb][sb] = cfrag<T>(gg);
                }
                rsum = sum_groups(rsum);
                if (g == 0) redk[w * TT + sb * 16 + lc] = rsum;
            }
#pragma unroll
            for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
                for (int sb = 0; sb < NTB; ++sb) {
                    f4 acc = f4zero();
                    mma_range<T>(acc, 0, NFB, [&](int fb) { return wt[eb][fb]; }, [&](int fb) { return gk[fb][sb]; });
                    *reinterpret_cast<f4 *>(red + (w * TT + sb * 16 + lc) * C::LDR + eb * 16 + 4 * g) = acc;
                }
            __syncthreads();
            reduce_rows<C>(red, nv, [&](int s, int e, f4 v, bool ok) {
                if (!ok) return;
                float rsum = redk[s];
#pragma unroll
                for (int ww = 1; ww < C::NW; ++ww) rsum += redk[ww * TT + s];
                const f4 kk = load4<T>(xk + s * C::LDX + e);
                store4<T>(dK + (size_t)(t0 + s) * D + e, v - kk * rsum);
            });
        } else {
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
                for (int sb = 0; sb < NTB; ++sb) {
                    const int s = sb * 16 + lc;
                    const f4 x = frag_to_f4<T>(lds_frag<T>(xk, C::LDX, sb * 16, w * MW + fb * 16));
                    f4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = dk[fb][sb][j] * elu1_grad(x[j]);
                    if (s < nv) store4<T>(dK + (size_t)(t0 + s) * D + w * MW + fb * 16 + 4 * g, v);
                }
        }
        // gradient state: dR += dNum^T g(Q), dS += sum dden g(Q) (after use)
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb) {
#pragma unroll
            for (int eb = 0; eb < NEB; ++eb) {
                mma_range<T>(dr[eb][fb], 0, NTB, [&](int tb) { return lds_frag<T>(dnt, C::LDT, eb * 16, tb * 16); },
                             [&](int tb) { return fqS[tb][fb]; });
                mma_range<T>(drt[fb][eb], 0, NTB, [&](int tb) { return fqS[tb][fb]; },
                             [&](int tb) { return lds_frag<T>(dnt, C::LDT, eb * 16, tb * 16); });
            }
            float s = 0.f;
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                const f4 q4 = frag_to_f4<T>(fqS[tb][fb]);
#pragma unroll
                for (int j = 0; j < 4; ++j) s += q4[j] * ddl[tb * 16 + 4 * g + j];
            }
            s = sum_groups(s);
            if (g == 0) dSl[w * MW + fb * 16 + lc] += s;
        }
        __syncthreads();
    }
}

}  // namespace slim
