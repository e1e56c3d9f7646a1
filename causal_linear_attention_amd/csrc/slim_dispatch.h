// slim_dispatch.h -- per-shape kernel tables (internal to libslim).
#pragma once
#include <hip/hip_runtime.h>
#include "slim_decode.h"
#include "slim_dw.h"

namespace slim {

struct KernelTable {
    int nt;  // threads per workgroup
    int tt;  // rows per tile
    // workgroups the chip holds at once (256 CUs) of the forward, dQ and dK/dV kernels
    // (their occupancy: waves per SIMD and LDS per CU)
    int slots_fwd, slots_q, slots_kv;
    void (*featmap)(dim3, hipStream_t, const void *, const void *, float *, float *, long long);
    void (*state)(dim3, hipStream_t, const ChunkArgs &);
    void (*fwd)(dim3, hipStream_t, const ChunkArgs &);
    void (*stats)(dim3, hipStream_t, const ChunkArgs &);
    // the row statistics from the forward's output and row records; NULL: the dQ
    // kernel makes them itself when ChunkArgs::Yin is set
    void (*rowstat)(dim3, hipStream_t, const ChunkArgs &);
    void (*gstate)(dim3, hipStream_t, const ChunkArgs &);  // NULL: the dQ kernel does its work
    void (*bwdq)(dim3, hipStream_t, const ChunkArgs &);
    void (*bwdkv)(dim3, hipStream_t, const ChunkArgs &);
    void (*decode)(dim3, hipStream_t, const DecodeArgs &, bool);  // bool: fp64 state
};

// The dW pass (FAVOR+): dQ and dK/dV kernels that also store dg(X) . g(X), and the
// row contraction that turns it into partial sums of dW.
struct DwTable {
    void (*bwdq)(dim3, hipStream_t, const ChunkArgs &);
    void (*bwdkv)(dim3, hipStream_t, const ChunkArgs &);
    void (*dw)(dim3, hipStream_t, const DwArgs &);
};

// One lookup per (dtype, feature map) translation unit; NULL if the shape is not compiled.
const KernelTable *table_f32_favor(int D, int M);
const KernelTable *table_bf16_favor(int D, int M);
const KernelTable *table_f32_elu1(int D, int M);
const KernelTable *table_bf16_elu1(int D, int M);
const DwTable *table_f32_favor_dw(int D, int M);
const DwTable *table_bf16_favor_dw(int D, int M);

}  // namespace slim
