// slim_dw.h -- gradient of the FAVOR+ projection W, which every batch row and
// head shares (page "Sub-Linear Memory: How to Make Performers SLiM",
// Subsection 2.1: g is the positive random feature map; the page keeps W fixed,
// this is the gradient a caller that trains it needs).
//
// g(x)_m = exp(w_m.x - |x|^2/2)/sqrt(M) depends on W only through w_m, with
// d g_m / d w_m = g_m x, so with dg the gradient w.r.t. the features
//     dW = sum over query rows of (dg(Q) . g(Q))^T Q + the same over key rows.
// The dQ and dK/dV kernels already form dg(X) . g(X) (their dQ, dK products
// contract it with W); in the dW pass they also store it, in the MFMA operand
// type, for the rows of the current window.  dw_kernel contracts it with the
// inputs over rows on the matrix cores: each workgroup sums a contiguous range
// of one head's rows into an [M][d] fp32 partial; sum_rows_kernel (in the host
// file) adds the partials in a fixed order, so the result is deterministic.
// Any positive per-row factor on g(Q) (the query offset) cancels in
// dg(Q) . g(Q), so the stored products are exact whatever offset was used.
#pragma once
#include "slim_device.h"

namespace slim {

struct DwArgs {
    const void *P[2];  // dg(Q).g(Q), dg(K).g(K): row r of head bh at (bh * prows + r) * M
    const void *X[2];  // Q, K [BH][L][d]: row r of the window at (bh * L + r0 + r) * d
    float *part;       // [2][BH][S][M][d] fp32 partial sums
    long long L;
    long long r0;      // first sequence row of the window
    long long prows;   // buffer rows per head
    int wl;            // rows of the window, per head
    int rps;           // rows per workgroup (a multiple of DW_TT)
    int S;             // workgroups per head and side
};

constexpr int DW_NT = 256;
constexpr int DW_TT = 32;

// grid (S, BH, 2): workgroup (s, bh, z) sums rows [s*rps, min(wl, (s+1)*rps)) of
// head bh, z = 0 for the query side, 1 for the key side.  Each wave owns a fixed
// set of the M/16 x d/16 output blocks; tiles of DW_TT rows are staged through LDS
// (the next tile's loads in flight during the current tile's products).
template <typename T, int D, int M> __global__ __launch_bounds__(DW_NT) void dw_kernel(DwArgs a)
{
    constexpr int NW = DW_NT / 64, TT = DW_TT, NTB = TT / 16;
    constexpr int NEB = D / 16, NBLK = (M / 16) * NEB, BPW = (NBLK + NW - 1) / NW;
    typedef LMat<T, TT, M, 32> PMat;  // rows t, cols m
    typedef LMat<T, TT, D, 32> XMat;  // rows t, cols e
    __shared__ __align__(16) T sp[PMat::SIZE];
    __shared__ __align__(16) T sx[XMat::SIZE];
    const PMat Pt(sp);
    const XMat Xt(sx);
    const int z = blockIdx.z, bh = blockIdx.y, s = blockIdx.x, w = wave_id();
    const int rb = s * a.rps;
    const int re = min(a.wl, rb + a.rps);
    const T *P = (const T *)a.P[z] + (size_t)bh * a.prows * M;
    const T *X = (const T *)a.X[z] + ((size_t)bh * a.L + a.r0) * D;
    f4 acc[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) acc[i] = f4zero();
    TileRegs<T, M, TT, DW_NT> rp;
    TileRegs<T, D, TT, DW_NT> rx;
    if (rb < re) {
        rp.load(P + (size_t)rb * M, re - rb);
        rx.load(X + (size_t)rb * D, re - rb);
    }
    for (int r = rb; r < re; r += TT) {
        rp.store(Pt, false, nullptr);
        rx.store(Xt, false, nullptr);
        __syncthreads();
        if (r + TT < re) {
            rp.load(P + (size_t)(r + TT) * M, re - r - TT);
            rx.load(X + (size_t)(r + TT) * D, re - r - TT);
        }
        // dW block (rows m, cols e) += sum_t P[t][m] X[t][e]; rows past the range are zero
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
            const int blk = w + NW * i;
            if (blk < NBLK) {
                const int mb = blk / NEB, eb = blk % NEB;
                mma_range<T>(acc[i], 0, NTB, [&](int tb) { return Pt.frag_r(mb * 16, tb * 16); },
                             [&](int tb) { return Xt.frag_r(eb * 16, tb * 16); });
            }
        }
        __syncthreads();
    }
    float *out = a.part + (((size_t)z * gridDim.y + bh) * a.S + s) * (size_t)(M * D);
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
        const int blk = w + NW * i;
        if (blk < NBLK) {
            const int mb = blk / NEB, eb = blk % NEB;
#pragma unroll
            for (int j = 0; j < 4; ++j) out[(size_t)(mb * 16 + 4 * lgrp() + j) * D + eb * 16 + lcol()] = acc[i][j];
        }
    }
}

}  // namespace slim
