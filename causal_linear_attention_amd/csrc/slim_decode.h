// slim_decode.h -- the recurrent decode step: one new token per (batch, head)
// advances the attention state and emits its output.  This is the iterative
// prefix-sum evaluation of page "Sub-Linear Memory: How to Make Performers
// SLiM", Subsection 2.1 (eq. (3)-(4)), taken one position at a time:
//
//     R' = R + v g(k)^T,   S' = S + g(k),   y = R' g(q) / (S' . g(q)).
//
// It is bound by streaming the (d+1) x M fp32 state [R; S] in and out once, so
// it is laid out for that and not for the matrix cores: one 256-thread
// workgroup per head; each thread owns four consecutive features of every
// (1024/M)-th state row, so rows move as contiguous 16-byte accesses.  The
// state loads are issued first and overlap the feature computation; g(k) and
// the query projection are computed once per workgroup (one feature per
// thread) and shared through LDS.  The numerators and the denominator are
// reduced over the M/4 threads of a row with lane shuffles.  At 545 MB of
// state this runs at 95% of the rate of a plain device copy of the same bytes;
// a persistent variant keeping W in registers across heads was no faster.
#pragma once
#include "slim_kernels.h"

namespace slim {

struct DecodeArgs {
    const void *q, *k, *v, *W;  // [BH][d] io dtype; W [M][d] (FAVOR+) or NULL
    const void *Rin, *Sin;      // state before the token (fp32 or fp64), NULL = zero
    void *y;                    // [BH][d] io dtype
    void *Rout, *Sout;          // state after the token (may equal Rin, Sin)
};

constexpr int DECODE_NT = 256;

// Four consecutive state entries of type S (fp32: 16 bytes, fp64: 32 bytes).
template <typename S> struct State4;
template <> struct State4<float> { typedef f4 type; };
template <> struct State4<double> { typedef double type __attribute__((ext_vector_type(4))); };

// S: the state's element type.  The features are fp32; with an fp64 state the update,
// the row dot products and the division are done in fp64.
template <class C, typename S> __global__ __launch_bounds__(DECODE_NT) void decode_kernel(DecodeArgs a)
{
    typedef typename C::T T;
    typedef typename State4<S>::type S4;
    constexpr int D = C::D, M = C::M;
    constexpr int TPR = M / 4;                       // threads per state row
    constexpr int RPP = DECODE_NT / TPR;             // rows per pass of the workgroup
    constexpr int NP = (D + 1 + RPP - 1) / RPP;      // passes over the D + 1 rows
    constexpr int NWF = (M + 63) / 64;               // waves that compute features
    static_assert(M % 16 == 0 && M <= DECODE_NT, "decode feature count");
    __shared__ float x[3][D];                        // q, k, v
    __shared__ float fk[M], pq[M];                   // g(k) (FAVOR+: its exponent); w_m.q (FAVOR+) or g(q) (elu+1)
    __shared__ float wmax[NWF], nmax[NWF];           // per wave: max_m w_m.q, max_m |w_m|^2
    __shared__ S red[D + 1];                         // numerators, then the denominator
    const long long bh = blockIdx.x;
    const int tid = threadIdx.x, cg = tid % TPR, rs = tid / TPR;
    const S *rin = a.Rin ? (const S *)a.Rin + (size_t)bh * D * M : nullptr;
    const S *sin_ = a.Sin ? (const S *)a.Sin + (size_t)bh * M : nullptr;
    S *rout = (S *)a.Rout + (size_t)bh * D * M;
    S *sout = (S *)a.Sout + (size_t)bh * M;

    S4 st[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int row = rs + p * RPP;
        st[p] = S4{0, 0, 0, 0};
        if (rin && row <= D)
            st[p] = *reinterpret_cast<const S4 *>((row < D ? rin + (size_t)row * M : sin_) + 4 * cg);
    }
    for (int i = tid; i < 3 * D; i += DECODE_NT) {
        const T *src = (const T *)(i < D ? a.q : i < 2 * D ? a.k : a.v);
        x[i / D][i % D] = (float)src[bh * D + i % D];
    }
    __syncthreads();

    if constexpr (C::FAVOR) {
        float qm = -__builtin_inff(), nn = 0.f;
        if (tid < M) {
            typedef typename Vec16<T>::type VT;
            constexpr int VN = Vec16<T>::N;
            const VT *w = reinterpret_cast<const VT *>((const T *)a.W + (size_t)tid * D);
            float sk = 0.f, sq = 0.f, kk = 0.f;
#pragma unroll 4
            for (int e0 = 0; e0 < D; e0 += VN) {
                const VT wv = w[e0 / VN];
#pragma unroll
                for (int j = 0; j < VN; ++j) {
                    const float we = (float)wv[j], ke = x[1][e0 + j];
                    sk = fmaf(we, ke, sk);
                    sq = fmaf(we, x[0][e0 + j], sq);
                    kk = fmaf(ke, ke, kk);
                    nn = fmaf(we, we, nn);  // |w_m|^2 in index order, as key_offset_block sums it
                }
            }
            // g(k)_m = exp(w_m.k - |k|^2/2 - koff) / sqrt(M): its exponent (base 2) here,
            // the key-side offset koff of W once the maximum of |w_m|^2 is known
            const float kn2 = (0.5f * kk + 0.5f * __logf((float)M)) * LOG2E;
            fk[tid] = fmaf(sk, LOG2E, -kn2);
            pq[tid] = sq;
            qm = sq;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            qm = fmaxf(qm, __shfl_xor(qm, o, 64));
            nn = fmaxf(nn, __shfl_xor(nn, o, 64));
        }
        if (tid < M && lane_id() == 0) {
            wmax[wave_id()] = qm;
            nmax[wave_id()] = nn;
        }
    } else {
        if (tid < M) {
            fk[tid] = elu1(x[1][tid]);
            pq[tid] = elu1(x[0][tid]);
        }
    }
    __syncthreads();

    // g(q) of this thread's four features.  FAVOR+: scaled by exp(-(max_m w_m.q)) and
    // without the |q|^2/2 and sqrt(M) factors: y is invariant to any positive factor
    // on g(q), and the largest feature becomes 1.
    float gk[4], gq[4];
    float qoff = 0.f, koff2 = 0.f;
    if constexpr (C::FAVOR) {
        qoff = wmax[0];
        float n2 = nmax[0];
#pragma unroll
        for (int w = 1; w < NWF; ++w) {
            qoff = fmaxf(qoff, wmax[w]);
            n2 = fmaxf(n2, nmax[w]);
        }
        qoff *= -LOG2E;
        koff2 = fmaxf(0.f, 0.5f * n2 - KOFF_MARGIN) * LOG2E;  // the key-side offset of W (slim_device.h)
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        gk[j] = C::FAVOR ? __builtin_amdgcn_exp2f(fk[4 * cg + j] - koff2) : fk[4 * cg + j];
        gq[j] = C::FAVOR ? __builtin_amdgcn_exp2f(fmaf(pq[4 * cg + j], LOG2E, qoff)) : pq[4 * cg + j];
    }

#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int row = rs + p * RPP;
        S part = 0;
        if (row <= D) {
            const float c = row < D ? x[2][row] : 1.f;
            S4 r = st[p];
#pragma unroll
            for (int j = 0; j < 4; ++j) r[j] += (S)c * (S)gk[j];
            // streaming store: the new state is not read again in this step, so it need not
            // occupy the caches (8-9% faster at 545 MB of state)
            __builtin_nontemporal_store(r, reinterpret_cast<S4 *>((row < D ? rout + (size_t)row * M : sout) + 4 * cg));
            part = r[0] * (S)gq[0];
#pragma unroll
            for (int j = 1; j < 4; ++j) part += r[j] * (S)gq[j];
        }
        // every lane of a row's group takes the same branch above; the shuffles stay
        // outside it so that the whole wave executes them
#pragma unroll
        for (int o = 1; o < TPR; o <<= 1) part += __shfl_xor(part, o, 64);
        if (row <= D && cg == 0) red[row] = part;
    }
    __syncthreads();
    if (tid < D) ((T *)a.y)[bh * D + tid] = (T)(float)(red[tid] / red[D]);
}

}  // namespace slim
