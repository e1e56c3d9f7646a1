// slim_host.hip -- the C ABI of libslim (include/slim.h): host-side validation,
// workspace planning and the slice-window launch sequence, plus the two small
// shape-independent kernels (state scan, copy/zero).
//
// Launch sequence (page "Sub-Linear Memory: How to Make Performers SLiM"); the
// chunk kernels run one workgroup per group of G consecutive slices:
//   forward  (Subsection 3.2): for each window of P groups in order:
//       state -> forward prefix scan (carry = running final state) -> fwd
//   backward (Subsection 3.3): for each window in reverse order:
//       state -> entry states (one window: forward prefix from the initial
//       state, or the forward's when the caller kept them; several: the window's
//       start state recovered from the state after it by subtraction, update (19)
//       at window granularity, then a forward prefix) -> stats (recompute
//       forward, per-row statistics; when the caller kept the forward's output
//       and row records, made from them by the dQ kernel itself or by a pass of
//       their own, rowstat) -> dQ
//       -> gstate (the slice's gradient w.r.t. its entry state; folded into the
//       dQ kernel where its registers allow) -> gradient suffix scan (update
//       (20)) -> dK, dV.  With several windows, a forward
//       sweep over all chunk contributions first rebuilds the final state.
//       dW pass: the dQ and dK/dV kernels also store dg(X) . g(X) for the
//       window's rows; each window ends with their contraction with Q and K
//       (dw) and the fixed-order sum of its partials into dW.
// All carries are fp64.
// The decode step (one token per head, Subsection 2.1's iterative evaluation) is
// a single kernel with no workspace.
// Only the carries (d x M + M per head) live across windows, so the workspace
// is bounded by the window, not by L.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/slim.h"
#include "slim_dispatch.h"

namespace slim {

// Kernel timing (diagnostics): when enabled, each launch below is bracketed by
// a pair of hipEvents recorded on the launch stream; slim_prof_entry() waits
// for the pending pairs and accumulates elapsed time per kernel name.
namespace prof {
struct Pending {
    std::string name;
    hipEvent_t a, b;
};
struct Total {
    double ms = 0.0;
    long long n = 0;
};
static std::mutex mu;
static bool on = false;
static std::vector<Pending> pending;
static std::vector<hipEvent_t> pool;
static std::map<std::string, Total> totals;
static std::vector<std::string> order;

static hipEvent_t take()
{
    if (!pool.empty()) {
        hipEvent_t e = pool.back();
        pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

struct Scope {
    bool active = false;
    Pending p;
    hipStream_t s;
    Scope(const char *name, hipStream_t st) : s(st)
    {
        std::lock_guard<std::mutex> g(mu);
        if (!on) return;
        p.name = name;
        p.a = take();
        p.b = take();
        if (!p.a || !p.b) return;
        active = hipEventRecord(p.a, s) == hipSuccess;
    }
    ~Scope()
    {
        if (!active) return;
        std::lock_guard<std::mutex> g(mu);
        hipEventRecord(p.b, s);
        pending.push_back(p);
    }
};

static void collect()
{
    for (auto &p : pending) {
        float ms = 0.f;
        if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
            if (!totals.count(p.name)) order.push_back(p.name);
            Total &t = totals[p.name];
            t.ms += ms;
            t.n += 1;
        }
        pool.push_back(p.a);
        pool.push_back(p.b);
    }
    pending.clear();
}
}  // namespace prof

#define SLIM_TIMED(name, s, call) \
    do {                          \
        prof::Scope _ps(name, s); \
        call;                     \
    } while (0)

__global__ __launch_bounds__(256) void copy_or_zero_kernel(float *dst, const float *src, long long n)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

static void copy_or_zero(float *dst, const float *src, long long n, hipStream_t s)
{
    if (n <= 0) return;
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dst, src, n);
}

// out[y][x] = (acc ? out[y][x] : 0) + sum of in[p][x] over rows p of block y
// (p = y*per .. min(rows, (y+1)*per) - 1, in increasing order), x < n4, in f4
// units: the fixed-order reduction of the dW partial sums.
__global__ __launch_bounds__(256) void sum_rows_kernel(const f4 *in, int rows, int n4, int per, f4 *out, int acc)
{
    const int x = blockIdx.x * 256 + threadIdx.x;
    if (x >= n4) return;
    const int p0 = blockIdx.y * per, p1 = min(rows, p0 + per);
    f4 *o = out + (size_t)blockIdx.y * n4 + x;
    f4 sum = acc ? *o : f4zero();
#pragma unroll 8
    for (int p = p0; p < p1; ++p) sum += in[(size_t)p * n4 + x];
    *o = sum;
}

// fp64 carries: loaded from a state of the caller's type (or zero), stored back in
// that type (rounded when it is fp32).
// Two carries stored back in one launch (in the caller's state type).
template <typename S>
__global__ __launch_bounds__(256) void narrow2_kernel(S *d0, const double *s0, long long n0, S *d1, const double *s1,
                                                      long long n1)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n0)
        d0[i] = (S)s0[i];
    else if (i - n0 < n1)
        d1[i - n0] = (S)s1[i - n0];
}
// Up to four carries loaded in one launch (each from its source, or zero).  The
// same launch's first workgroup computes the key-side offset of W (FAVOR+) into the
// workspace and, if wanted, the caller's koff (0 for elu+1, which has no W).
struct WidenSet {
    double *dst[4];
    const void *src[4];
    long long n[4];
    const void *W;  // FAVOR+ projection [M][D], or NULL
    int wbf16, M, D;
    float *kws, *kout;  // key offset: workspace copy (read by the chunk kernels), caller's copy
};
template <typename S> __global__ __launch_bounds__(256) void widen_set_kernel(WidenSet w)
{
    if (blockIdx.x == 0) {
        __shared__ float red[5];
        float koff = 0.f;
        if (w.W) koff = key_offset_block(w.W, w.wbf16, w.M, w.D, red);
        if (threadIdx.x == 0) {
            if (w.kws) *w.kws = koff;
            if (w.kout) *w.kout = koff;
        }
    }
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (i < w.n[k]) {
            w.dst[k][i] = w.src[k] ? (double)((const S *)w.src[k])[i] : 0.0;
            return;
        }
        i -= w.n[k];
    }
}
static void widen(const WidenSet &w, bool f64, hipStream_t s)
{
    const long long n = w.n[0] + w.n[1] + w.n[2] + w.n[3];
    if (n <= 0 && !w.kws && !w.kout) return;
    const dim3 g((unsigned)(n > 0 ? (n + 255) / 256 : 1));
    if (f64)
        hipLaunchKernelGGL(widen_set_kernel<double>, g, dim3(256), 0, s, w);
    else
        hipLaunchKernelGGL(widen_set_kernel<float>, g, dim3(256), 0, s, w);
}
static void narrow2(void *d0, const double *s0, long long n0, void *d1, const double *s1, long long n1, bool f64,
                    hipStream_t s)
{
    const long long n = n0 + n1;
    if (n <= 0) return;
    const dim3 g((unsigned)((n + 255) / 256));
    if (f64)
        hipLaunchKernelGGL(narrow2_kernel<double>, g, dim3(256), 0, s, (double *)d0, s0, n0, (double *)d1, s1, n1);
    else
        hipLaunchKernelGGL(narrow2_kernel<float>, g, dim3(256), 0, s, (float *)d0, s0, n0, (float *)d1, s1, n1);
}

// Fragment-packed W^T: for value block eb and feature block mb, lane i of a
// wave reads 4 consecutive elements W[mb*16 + 4(i/16) + j][eb*16 + i%16] at
// Wp[((eb*(M/16) + mb)*64 + i)*4 + j]  (elements of 2 or 4 bytes moved as integers).
template <typename U> __global__ __launch_bounds__(256) void pack_wt_kernel(const U *W, U *Wp, int M, int D)
{
    const int o = blockIdx.x * 256 + threadIdx.x;
    if (o >= M * D) return;
    const int j = o & 3, i = (o >> 2) & 63, blk = o >> 8;
    const int mb = blk % (M / 16), eb = blk / (M / 16);
    Wp[o] = W[(size_t)(mb * 16 + 4 * (i / 16) + j) * D + eb * 16 + i % 16];
}

static void pack_wt(const void *W, void *Wp, int M, int D, bool bf16, hipStream_t s)
{
    const dim3 grid((unsigned)((M * D + 255) / 256));
    if (bf16)
        hipLaunchKernelGGL(pack_wt_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t *)W, (uint16_t *)Wp, M, D);
    else
        hipLaunchKernelGGL(pack_wt_kernel<uint32_t>, grid, dim3(256), 0, s, (const uint32_t *)W, (uint32_t *)Wp, M, D);
}

// scan_kernel lives in slim_kernels.h (instantiated here once).
static void scan(int mode, float *slots, double *cR, double *cS, int D, int M, int P, int np, int BH, hipStream_t s)
{
    const int SZ = (D + 1) * M;
    const long long elems = (long long)(SZ / 4) * BH;
    // segments of the chunk range: enough workgroups to fill the chip (about 1024),
    // at least 4 chunks per segment, at most 32 segments
    int G = 1;
    while (G < 32 && elems * G < 1024LL * 256 && np >= 8 * G) G *= 2;
    const int E = 256 / G;
    dim3 grid((unsigned)((SZ / 4 + E - 1) / E), (unsigned)BH);
    static const char *names[4] = {"scan_prefix", "scan_window", "scan_grad", "scan_sum"};
    prof::Scope ps(names[mode], s);
    // a totals pass over segments short enough to keep in registers: the variant that
    // reads each slot once (at 1M tokens x 8 heads in 1024 groups, 0.068 -> 0.051 ms);
    // not for segments of a few slots, which it slows (0.008 -> 0.012 ms at 8 slots)
    const int sl = (np + G - 1) / G;
    const bool keep = (mode == 1 || mode == 3 || G > 1) && sl > 8 && sl <= SCAN_KEEP;
    typedef void (*ScanFn)(float *, double *, double *, int, int, int, int, int);
    static const ScanFn fns[4][2] = {{scan_kernel<0, false>, scan_kernel<0, true>},
                                     {scan_kernel<1, false>, scan_kernel<1, true>},
                                     {scan_kernel<2, false>, scan_kernel<2, true>},
                                     {scan_kernel<3, false>, scan_kernel<3, true>}};
    hipLaunchKernelGGL(fns[mode][keep ? 1 : 0], grid, dim3(256), 0, s, slots, cR, cS, D * M, M, P, np, G);
}

static const KernelTable *find(const slim_desc *d)
{
    if (d->d > 1024 || d->M > 1024) return nullptr;
    const int D = (int)d->d, M = (int)d->M;
    if (d->dtype == SLIM_F32) return d->feat == SLIM_FEAT_FAVOR ? table_f32_favor(D, M) : table_f32_elu1(D, M);
    return d->feat == SLIM_FEAT_FAVOR ? table_bf16_favor(D, M) : table_bf16_elu1(D, M);
}

static const DwTable *find_dw(const slim_desc *d)
{
    if (d->feat != SLIM_FEAT_FAVOR || d->d > 1024 || d->M > 1024) return nullptr;
    const int D = (int)d->d, M = (int)d->M;
    return d->dtype == SLIM_F32 ? table_f32_favor_dw(D, M) : table_bf16_favor_dw(D, M);
}

struct Plan {
    long long BH;
    long long G;        // slices per group: one workgroup walks G consecutive slices
    long long c;        // rows per group (G slices, at most L)
    long long nchunks;  // groups
    long long P;        // groups per window
    long long SZ;
    long long dw_parts;  // dW pass: partial sums per window (2 sides x BH x workgroups per head)
    size_t slots_off, gslots_off, stats_off, cR_off, cS_off, gR_off, gS_off, wt_off, koff_off;
    size_t pq_off, pk_off, part_off, part2_off;
    size_t total;         // workspace bytes
    size_t total_states;  // workspace bytes when the caller holds the slices' states (the
                          // slot array is the last region; equal to total for several windows)
    bool one_window() const { return P == nchunks; }
};

// dW pass: the row contraction runs about 1024 workgroups (at least 256 rows each).
// dw_groups: the target workgroups per head and side for wl rows (non-decreasing in
// wl); dw_split: the split actually used, S <= dw_groups workgroups of rows_per rows.
static long long dw_groups(long long BH, long long wl)
{
    long long s = (1024 + 2 * BH - 1) / (2 * BH);
    const long long smax = (wl + 255) / 256;
    if (s > smax) s = smax;
    return s < 1 ? 1 : s;
}
static void dw_split(long long BH, long long wl, int *S, int *rows_per)
{
    const long long s = dw_groups(BH, wl);
    long long rp = (wl + s - 1) / s;
    rp = (rp + DW_TT - 1) / DW_TT * DW_TT;
    *rows_per = (int)rp;
    *S = (int)((wl + rp - 1) / rp);
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Automatic window: enough slices for about 4096 workgroups per launch; all of them
// when the backward's per-slice buffers for the whole sequence fit the budget, so that
// it runs as one window (no extra sweep over the slices, no recompute of their states
// per window); and never more slices than fit it (at least one).  The budget is 1 GiB
// for the state and gradient slots with the row statistics, and with dW another 1 GiB
// for its two [c][M] rows of dg(X) . g(X) per slice and head.  The workspace is
// therefore bounded for any L at a given slice length.
constexpr long long WINDOW_BUDGET = 1LL << 30;
static long long resolve_window(const slim_desc *d, long long nchunks, long long c, long long G, int pass)
{
    long long P = d->window_chunks > 0 ? (d->window_chunks / G > 0 ? d->window_chunks / G : 1) : 0;
    if (P <= 0) {
        const long long BH = d->B * d->H;
        const long long per_state = BH * ((d->d + 1) * d->M * 4 * 2 + c * ROWSTAT * 4);
        const long long per_dw = pass == SLIM_PASS_BWD_DW ? BH * 2 * c * d->M * (d->dtype == SLIM_BF16 ? 2 : 4) : 0;
        long long most = WINDOW_BUDGET / per_state;  // slices that fit the budgets
        if (per_dw > 0 && WINDOW_BUDGET / per_dw < most) most = WINDOW_BUDGET / per_dw;
        P = (4096 + BH - 1) / BH;
        if (nchunks > P && nchunks <= most) P = nchunks;
        if (P > most) P = most;
    }
    if (P > nchunks) P = nchunks;
    if (P < 1) P = 1;
    if (P > 65535) P = 65535;
    return P;
}

// Slices per group: the chunk kernels run one workgroup per group of G consecutive
// slices, walking them in order and carrying the state from one slice to the next (the
// slice loop of Subsection 3.2, G slices at a time), so that one state per group is
// written, scanned and read back, and a workgroup's start-up (loading its entry state)
// is paid once per group.  Automatic: the largest G, a power of two with groups of at
// most 2048 rows, whose launches still fill the chip in whole rounds, within 10%, for
// each of the forward, dQ and dK/dV kernels: at least as many workgroups as the chip
// holds of that kernel at once (its slots: 512 for two 4-wave workgroups per CU, 768
// for the dQ kernel's three at bf16, M = 64, ...), and workgroups / (rounds x slots)
// >= 0.9.  Measured step times (fwd+bwd, forward states kept):
// 16K tokens x 64 heads in slices of 512, G = 1, 2, 4, 8: 1.45, 1.35, 1.29, 1.72 ms
// (4: 512 workgroups, one round; 8 leaves half the chip idle); elu+1 at d = M = 128,
// 8K tokens x 96 heads in slices of 256: 1.32, 1.17, 1.21, 1.43 ms (4: 768 workgroups,
// a second round half empty); 1M tokens x 8 heads in slices of 512: 4.81, 4.55, 4.57,
// 4.52 ms (at 8 the dQ kernel's last round of 768 is two-thirds full: 1.44 -> 1.53 ms).
// Few heads and slices (under 512 workgroups even at G = 1): 1.
static long long group_of(const slim_desc *d, long long nslices, long long c)
{
    if (d->group_slices > 0) return d->group_slices < nslices ? d->group_slices : nslices;
    const KernelTable *kt = find(d);
    if (!kt) return 1;
    const long long BH = d->B * d->H;
    auto fills = [](long long wgs, long long slots) {
        const long long rounds = (wgs + slots - 1) / slots;
        return wgs >= slots && 10 * wgs >= 9 * rounds * slots;
    };
    long long best = 1;
    for (long long G = 1; G <= nslices && G * c <= 2048; G *= 2) {
        const long long wgs = (nslices + G - 1) / G * BH;
        if (fills(wgs, kt->slots_fwd) && fills(wgs, kt->slots_q) && fills(wgs, kt->slots_kv)) best = G;
    }
    return best;
}

// window > 0: hold that many groups per window instead of the resolved window.
static Plan plan(const slim_desc *d, int pass, long long window = 0)
{
    Plan p;
    memset(&p, 0, sizeof(p));
    p.BH = d->B * d->H;
    const long long cs = (d->L + d->num_chunks - 1) / d->num_chunks;  // rows per slice
    p.G = group_of(d, (d->L + cs - 1) / cs, cs);
    p.c = cs * p.G < d->L ? cs * p.G : d->L;
    p.nchunks = (d->L + p.c - 1) / p.c;
    p.P = window > 0 ? (window < p.nchunks ? window : p.nchunks) : resolve_window(d, p.nchunks, p.c, p.G, pass);
    p.SZ = (d->d + 1) * d->M;
    const size_t slots = (size_t)p.BH * (p.P + 1) * p.SZ * 4;
    size_t off = 0;
    // fp64 carries of the state (both passes) and of its gradient (backward)
    p.cR_off = off;
    off = align256(off + (size_t)p.BH * d->d * d->M * 8);
    p.cS_off = off;
    off = align256(off + (size_t)p.BH * d->M * 8);
    p.koff_off = off;  // the key-side offset of W, one float
    off = align256(off + 4);
    if (pass == SLIM_PASS_BWD || pass == SLIM_PASS_BWD_DW) {
        p.gslots_off = off;
        off = align256(off + slots);
        p.stats_off = off;
        off = align256(off + (size_t)p.BH * p.P * p.c * ROWSTAT * 4);
        p.gR_off = off;
        off = align256(off + (size_t)p.BH * d->d * d->M * 8);
        p.gS_off = off;
        off = align256(off + (size_t)p.BH * d->M * 8);
        if (d->feat == SLIM_FEAT_FAVOR) {  // fragment-packed W^T (coalesced fragment loads)
            p.wt_off = off;
            off = align256(off + (size_t)d->d * d->M * (d->dtype == SLIM_BF16 ? 2 : 4));
        }
    }
    if (pass == SLIM_PASS_BWD_DW) {
        // dg(X) . g(X) of the window's rows for queries and keys, in the operand type
        const size_t pbytes = (size_t)p.BH * p.P * p.c * d->M * (d->dtype == SLIM_BF16 ? 2 : 4);
        p.pq_off = off;
        off = align256(off + pbytes);
        p.pk_off = off;
        off = align256(off + pbytes);
        // every window has at most min(P c, L) rows, so at most this many partials
        p.dw_parts = 2 * p.BH * dw_groups(p.BH, p.P * p.c < d->L ? p.P * p.c : d->L);
        const size_t pmd = (size_t)d->M * d->d * 4;
        p.part_off = off;
        off = align256(off + (size_t)p.dw_parts * pmd);
        p.part2_off = off;
        off = align256(off + (size_t)((p.dw_parts + 31) / 32) * pmd);
    }
    // the state slots last: a call handed every slice's state by the caller (one
    // window) needs no room for them
    p.slots_off = off;
    const size_t without = off;
    off = align256(off + slots);
    const bool none = pass == SLIM_PASS_FEATMAP || pass == SLIM_PASS_DECODE;
    p.total = none ? 0 : off;
    p.total_states = none ? 0 : p.one_window() ? without : off;
    return p;
}

static bool misaligned(const void *p, uintptr_t a) { return p && ((uintptr_t)p % a) != 0; }

// Two ranges of n bytes that overlap without being the same range.
static bool overlaps_partly(const void *x, const void *y, long long n)
{
    if (!x || !y || x == y) return false;
    const char *a = (const char *)x, *b = (const char *)y;
    return a < b + n && b < a + n;
}

}  // namespace slim

using namespace slim;

extern "C" {

int slim_version(void) { return (4 << 16) | 0; }

slim_status slim_prof_enable(int enable)
{
    std::lock_guard<std::mutex> g(prof::mu);
    prof::collect();
    if (enable) {
        prof::totals.clear();
        prof::order.clear();
    }
    prof::on = enable != 0;
    return SLIM_OK;
}

int slim_prof_count(void)
{
    std::lock_guard<std::mutex> g(prof::mu);
    prof::collect();
    return (int)prof::order.size();
}

slim_status slim_prof_entry(int i, const char **name, double *total_ms, int64_t *launches)
{
    std::lock_guard<std::mutex> g(prof::mu);
    prof::collect();
    if (i < 0 || i >= (int)prof::order.size()) return SLIM_ERR_SHAPE;
    if (!name || !total_ms || !launches) return SLIM_ERR_NULL;
    const prof::Total &t = prof::totals[prof::order[i]];
    *name = prof::order[i].c_str();
    *total_ms = t.ms;
    *launches = t.n;
    return SLIM_OK;
}

const char *slim_status_string(slim_status s)
{
    switch (s) {
    case SLIM_OK: return "ok";
    case SLIM_ERR_NULL: return "required pointer is NULL";
    case SLIM_ERR_SHAPE: return "shape or slice count out of range";
    case SLIM_ERR_DTYPE: return "unknown dtype or feature map";
    case SLIM_ERR_UNSUPPORTED: return "shape not supported by the compiled kernels";
    case SLIM_ERR_WORKSPACE: return "workspace too small";
    case SLIM_ERR_ALIGN: return "misaligned pointer";
    case SLIM_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

slim_status slim_validate(const slim_desc *d, int pass)
{
    if (!d) return SLIM_ERR_NULL;
    if (d->dtype != SLIM_F32 && d->dtype != SLIM_BF16) return SLIM_ERR_DTYPE;
    if (d->feat != SLIM_FEAT_FAVOR && d->feat != SLIM_FEAT_ELU1) return SLIM_ERR_DTYPE;
    if (pass < SLIM_PASS_FEATMAP || pass > SLIM_PASS_BWD_DW) return SLIM_ERR_SHAPE;
    if (d->B < 1 || d->H < 1 || d->L < 1 || d->d < 1 || d->M < 1) return SLIM_ERR_SHAPE;
    if (d->L >= (1LL << 31) || d->B > (1LL << 31) || d->H > (1LL << 31)) return SLIM_ERR_SHAPE;
    if (pass != SLIM_PASS_FEATMAP && (d->num_chunks < 1 || d->num_chunks > d->L)) return SLIM_ERR_SHAPE;
    if (d->window_chunks < 0 || d->group_slices < 0) return SLIM_ERR_SHAPE;
    if (d->feat == SLIM_FEAT_ELU1 && d->M != d->d) return SLIM_ERR_SHAPE;
    if (d->state_dtype != SLIM_F32 && d->state_dtype != SLIM_F64) return SLIM_ERR_DTYPE;
    if (pass == SLIM_PASS_DECODE && d->L != 1) return SLIM_ERR_SHAPE;
    const long long BH = d->B * d->H;
    if (pass == SLIM_PASS_DECODE ? BH > (1LL << 24) : (BH > 65535 && pass != SLIM_PASS_FEATMAP))
        return SLIM_ERR_UNSUPPORTED;
    if ((double)BH * (double)d->L * (double)(d->d > d->M ? d->d : d->M) > 4.0e18) return SLIM_ERR_SHAPE;
    if (!find(d)) return SLIM_ERR_UNSUPPORTED;
    if (pass == SLIM_PASS_BWD_DW && !find_dw(d)) return SLIM_ERR_UNSUPPORTED;  // FAVOR+ only
    return SLIM_OK;
}

size_t slim_workspace_bytes(const slim_desc *d, int pass)
{
    if (slim_validate(d, pass) != SLIM_OK) return 0;
    return plan(d, pass).total;
}

size_t slim_state_bytes(const slim_desc *d)
{
    if (slim_validate(d, SLIM_PASS_FWD) != SLIM_OK) return 0;
    const Plan p = plan(d, SLIM_PASS_FWD);
    return p.one_window() ? (size_t)p.BH * (p.nchunks + 1) * p.SZ * 4 : 0;
}

size_t slim_workspace_bytes_states(const slim_desc *d, int pass)
{
    if (slim_validate(d, pass) != SLIM_OK) return 0;
    return plan(d, pass).total_states;
}

int64_t slim_window_chunks(const slim_desc *d)
{
    if (slim_validate(d, SLIM_PASS_FWD) != SLIM_OK) return 0;
    const Plan p = plan(d, SLIM_PASS_FWD);
    const long long cs = (d->L + d->num_chunks - 1) / d->num_chunks, ns = (d->L + cs - 1) / cs;
    return p.P * p.G < ns ? p.P * p.G : ns;
}

int64_t slim_group_slices(const slim_desc *d)
{
    if (slim_validate(d, SLIM_PASS_FWD) != SLIM_OK) return 0;
    return plan(d, SLIM_PASS_FWD).G;
}

int64_t slim_tile_rows(const slim_desc *d)
{
    if (slim_validate(d, SLIM_PASS_FWD) != SLIM_OK) return 0;
    return find(d)->tt;
}

slim_status slim_featmap(const slim_desc *d, const void *X, const void *W, float *phi, float *row_offset,
                         void *stream)
{
    slim_status st = slim_validate(d, SLIM_PASS_FEATMAP);
    if (st != SLIM_OK) return st;
    if (!X || !phi) return SLIM_ERR_NULL;
    if (d->feat == SLIM_FEAT_FAVOR && !W) return SLIM_ERR_NULL;
    if (d->feat == SLIM_FEAT_ELU1 && (W || row_offset)) return SLIM_ERR_SHAPE;
    if (misaligned(X, 16) || misaligned(W, 16) || misaligned(phi, 16) || misaligned(row_offset, 4))
        return SLIM_ERR_ALIGN;
    const KernelTable *kt = find(d);
    const long long rows = d->B * d->H * d->L;
    const long long nblk = (rows + (long long)kt->tt * FEATMAP_TILES - 1) / ((long long)kt->tt * FEATMAP_TILES);
    if (nblk > 0x7fffffffLL) return SLIM_ERR_SHAPE;
    SLIM_TIMED("featmap", (hipStream_t)stream,
               kt->featmap(dim3((unsigned)nblk), (hipStream_t)stream, X, W, phi, row_offset, rows));
    return hipGetLastError() == hipSuccess ? SLIM_OK : SLIM_ERR_HIP;
}

}  // extern "C"

namespace slim {

// Argument checks shared by the two forward entry points (host only, no HIP call).
static slim_status check_fwd_args(const slim_desc *d, const void *Q, const void *K, const void *V, const void *W,
                                  const void *R_in, const void *S_in, const void *Y, const void *R_out,
                                  const void *S_out, const float *koff, const float *row_stats,
                                  const float *states = nullptr)
{
    slim_status st = slim_validate(d, SLIM_PASS_FWD);
    if (st != SLIM_OK) return st;
    if (!Q || !K || !V || !Y || !R_out || !S_out) return SLIM_ERR_NULL;
    if (d->feat == SLIM_FEAT_FAVOR && !W) return SLIM_ERR_NULL;
    if (d->feat == SLIM_FEAT_ELU1 && W) return SLIM_ERR_SHAPE;
    if ((R_in == nullptr) != (S_in == nullptr)) return SLIM_ERR_NULL;
    if (misaligned(Q, 16) || misaligned(K, 16) || misaligned(V, 16) || misaligned(W, 16) || misaligned(Y, 16) ||
        misaligned(R_out, 16) || misaligned(S_out, 16) || misaligned(R_in, 16) || misaligned(S_in, 16) ||
        misaligned(row_stats, 16) || misaligned(koff, 4) || misaligned(states, 16))
        return SLIM_ERR_ALIGN;
    return SLIM_OK;
}

// The forward's launch sequence over a workspace laid out by p (checked arguments).
static slim_status fwd_launch(const slim_desc *d, const Plan &p, const void *Q, const void *K, const void *V,
                              const void *W, const void *R_in, const void *S_in, void *Y, void *R_out, void *S_out,
                              float *koff, float *row_stats, float *states, char *base, hipStream_t s)
{
    const KernelTable *kt = find(d);
    const int D = (int)d->d, M = (int)d->M, BH = (int)p.BH;
    ChunkArgs a;
    memset(&a, 0, sizeof(a));
    a.Q = Q; a.K = K; a.V = V; a.W = W; a.out0 = Y;
    a.rstat = row_stats;
    a.slots = states ? states : (float *)(base + p.slots_off);  // the caller's: one window
    a.L = d->L; a.c = (int)p.c; a.P = (int)p.P;
    a.koff = (const float *)(base + p.koff_off);
    double *cR = (double *)(base + p.cR_off), *cS = (double *)(base + p.cS_off);
    const bool f64 = d->state_dtype == SLIM_F64;
    widen(WidenSet{{cR, cS, nullptr, nullptr},
                   {R_in, S_in, nullptr, nullptr},
                   {p.BH * D * M, p.BH * M, 0, 0},
                   W, d->dtype == SLIM_BF16, M, D, (float *)(base + p.koff_off), koff},
          f64, s);
    for (long long n0 = 0; n0 < p.nchunks; n0 += p.P) {
        const int np = (int)(p.nchunks - n0 < p.P ? p.nchunks - n0 : p.P);
        a.n0 = (int)n0;
        SLIM_TIMED("state", s, kt->state(dim3(np, BH), s, a));
        scan(0, a.slots, cR, cS, D, M, (int)p.P, np, BH, s);
        SLIM_TIMED("fwd", s, kt->fwd(dim3(np, BH), s, a));
    }
    narrow2(R_out, cR, p.BH * D * M, S_out, cS, p.BH * M, f64, s);
    return hipGetLastError() == hipSuccess ? SLIM_OK : SLIM_ERR_HIP;
}

// The allocation-free forward's workspace: one array per GPU the library runs on, held
// until the process ends.  Host code never uses this name as an address (on the host it
// is only a stand-in for the symbol): scratch_base() looks up each device's own copy
// with hipGetSymbolAddress once, with that device current, and keeps it.
constexpr size_t NOALLOC_SCRATCH_BYTES = SLIM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];
static std::mutex scratch_mu;
static std::vector<void *> scratch_ptr;  // per device ordinal; null until looked up

// The scratch array of the device that runs `s` (the current device for the null stream).
static hipError_t scratch_base(hipStream_t s, char **out)
{
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (s) {
        e = hipStreamGetDevice(s, &dev);
        if (e != hipSuccess) return e;
    }
    std::lock_guard<std::mutex> g(scratch_mu);
    if (dev < 0) return hipErrorInvalidDevice;
    if ((size_t)dev >= scratch_ptr.size()) scratch_ptr.resize(dev + 1, nullptr);
    if (!scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        scratch_ptr[dev] = p;
    }
    *out = (char *)scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace slim

extern "C" {

slim_status slim_attn_fwd(const slim_desc *d, const void *Q, const void *K, const void *V, const void *W,
                          const void *R_in, const void *S_in, void *Y, void *R_out, void *S_out, float *koff,
                          float *row_stats, float *states, void *ws, size_t ws_bytes, void *stream)
{
    slim_status st = check_fwd_args(d, Q, K, V, W, R_in, S_in, Y, R_out, S_out, koff, row_stats, states);
    if (st != SLIM_OK) return st;
    if (!ws) return SLIM_ERR_NULL;
    if (misaligned(ws, 256)) return SLIM_ERR_ALIGN;
    const Plan p = plan(d, SLIM_PASS_FWD);
    if (states && !p.one_window()) return SLIM_ERR_SHAPE;  // the states of every slice need one window
    if (ws_bytes < (states ? p.total_states : p.total)) return SLIM_ERR_WORKSPACE;
    return fwd_launch(d, p, Q, K, V, W, R_in, S_in, Y, R_out, S_out, koff, row_stats, states, (char *)ws,
                      (hipStream_t)stream);
}

slim_status slim_attn_fwd_noalloc(const slim_desc *d, const void *Q, const void *K, const void *V, const void *W,
                                  const void *R_in, const void *S_in, void *Y, void *R_out, void *S_out,
                                  float *koff, float *row_stats, void *stream)
{
    slim_status st = check_fwd_args(d, Q, K, V, W, R_in, S_in, Y, R_out, S_out, koff, row_stats);
    if (st != SLIM_OK) return st;
    // the resolved window, or (automatic window) the most slices that fit the scratch
    Plan p = plan(d, SLIM_PASS_FWD);
    if (p.total > NOALLOC_SCRATCH_BYTES) {
        if (d->window_chunks > 0) return SLIM_ERR_WORKSPACE;
        long long lo = 1, hi = p.P - 1;  // the plan's size grows with the window
        if (plan(d, SLIM_PASS_FWD, 1).total > NOALLOC_SCRATCH_BYTES) return SLIM_ERR_WORKSPACE;
        while (lo < hi) {
            const long long mid = (lo + hi + 1) / 2;
            if (plan(d, SLIM_PASS_FWD, mid).total <= NOALLOC_SCRATCH_BYTES)
                lo = mid;
            else
                hi = mid - 1;
        }
        p = plan(d, SLIM_PASS_FWD, lo);
    }
    char *base = nullptr;
    if (scratch_base((hipStream_t)stream, &base) != hipSuccess) return SLIM_ERR_HIP;
    return fwd_launch(d, p, Q, K, V, W, R_in, S_in, Y, R_out, S_out, koff, row_stats, nullptr, base,
                      (hipStream_t)stream);
}

slim_status slim_attn_bwd(const slim_desc *d, const void *Q, const void *K, const void *V, const void *W,
                          const void *dY, const void *Y, const float *row_stats, const float *states,
                          const void *R_in, const void *S_in, const void *dR_out, const void *dS_out, void *dQ,
                          void *dK, void *dV, void *dR_in, void *dS_in, float *dW, void *ws, size_t ws_bytes,
                          void *stream)
{
    const int pass = dW ? SLIM_PASS_BWD_DW : SLIM_PASS_BWD;
    slim_status st = slim_validate(d, pass);
    if (st != SLIM_OK) return st;
    if (!Q || !K || !V || !dY || !dQ || !dK || !dV || !ws) return SLIM_ERR_NULL;
    if (d->feat == SLIM_FEAT_FAVOR && !W) return SLIM_ERR_NULL;
    if (d->feat == SLIM_FEAT_ELU1 && W) return SLIM_ERR_SHAPE;
    if ((R_in == nullptr) != (S_in == nullptr)) return SLIM_ERR_NULL;
    if ((dR_out == nullptr) != (dS_out == nullptr)) return SLIM_ERR_NULL;
    if ((dR_in == nullptr) != (dS_in == nullptr)) return SLIM_ERR_NULL;
    if ((Y == nullptr) != (row_stats == nullptr)) return SLIM_ERR_NULL;
    if (misaligned(Y, 16) || misaligned(row_stats, 16) || misaligned(states, 16)) return SLIM_ERR_ALIGN;
    if (misaligned(Q, 16) || misaligned(K, 16) || misaligned(V, 16) || misaligned(W, 16) || misaligned(dY, 16) ||
        misaligned(R_in, 16) || misaligned(S_in, 16) || misaligned(dR_out, 16) || misaligned(dS_out, 16) ||
        misaligned(dQ, 16) || misaligned(dK, 16) || misaligned(dV, 16) || misaligned(dR_in, 16) ||
        misaligned(dS_in, 16) || misaligned(dW, 16) || misaligned(ws, 256))
        return SLIM_ERR_ALIGN;
    const Plan p = plan(d, pass);
    // the forward's states of every slice, used where this pass holds them all in one window
    // (else rebuilt as without them, to the same values)
    const bool kept = states && p.one_window();
    if (ws_bytes < (kept ? p.total_states : p.total)) return SLIM_ERR_WORKSPACE;
    const KernelTable *kt = find(d);
    const DwTable *dt = dW ? find_dw(d) : nullptr;
    hipStream_t s = (hipStream_t)stream;
    const int D = (int)d->d, M = (int)d->M, BH = (int)p.BH;
    char *base = (char *)ws;
    ChunkArgs a;
    memset(&a, 0, sizeof(a));
    a.Q = Q; a.K = K; a.V = V; a.W = W; a.dY = dY;
    a.Yin = Y; a.rstat = const_cast<float *>(row_stats);
    a.out0 = dQ; a.out1 = dK; a.out2 = dV;
    a.slots = kept ? const_cast<float *>(states) : (float *)(base + p.slots_off);  // read only when kept
    a.gslots = (float *)(base + p.gslots_off);
    a.stats = (float *)(base + p.stats_off);
    a.L = d->L; a.c = (int)p.c; a.P = (int)p.P;
    a.koff = (const float *)(base + p.koff_off);
    if (dt) {
        a.pq = base + p.pq_off;
        a.pk = base + p.pk_off;
    }
    double *cR = (double *)(base + p.cR_off), *cS = (double *)(base + p.cS_off);
    double *gR = (double *)(base + p.gR_off), *gS = (double *)(base + p.gS_off);
    if (d->feat == SLIM_FEAT_FAVOR) {
        a.Wt = base + p.wt_off;
        pack_wt(W, base + p.wt_off, M, D, d->dtype == SLIM_BF16, s);
    }
    const bool f64 = d->state_dtype == SLIM_F64;
    widen(WidenSet{{cR, cS, gR, gS},
                   {R_in, S_in, dR_out, dS_out},
                   {p.BH * D * M, p.BH * M, p.BH * D * M, p.BH * M},
                   W, d->dtype == SLIM_BF16, M, D, (float *)(base + p.koff_off), nullptr},
          f64, s);
    const long long nwin = (p.nchunks + p.P - 1) / p.P;
    auto window = [&](long long wi) {
        const long long n0 = wi * p.P;
        a.n0 = (int)n0;
        return (int)(p.nchunks - n0 < p.P ? p.nchunks - n0 : p.P);
    };
    if (nwin > 1) {
        // Several windows: the reverse walk needs the state after the last one.  It is
        // rebuilt here, in fp64, from the initial state and every chunk's contribution
        // (the fp32 final state of the forward would carry its rounding into every
        // entry state recovered from it by subtraction).
        for (long long wi = 0; wi < nwin; ++wi) {
            const int np = window(wi);
            SLIM_TIMED("state", s, kt->state(dim3(np, BH), s, a));
            scan(3, a.slots, cR, cS, D, M, (int)p.P, np, BH, s);
        }
    }
    for (long long wi = nwin - 1; wi >= 0; --wi) {
        const int np = window(wi);
        if (nwin == 1) {  // entry states forward from the initial state (unless the forward's are kept)
            if (!kept) {
                SLIM_TIMED("state", s, kt->state(dim3(np, BH), s, a));
                scan(0, a.slots, cR, cS, D, M, (int)p.P, np, BH, s);
            }
        } else {  // window start = state after it minus its chunks; entry states forward from there
            if (wi != nwin - 1) SLIM_TIMED("state", s, kt->state(dim3(np, BH), s, a));
            scan(1, a.slots, cR, cS, D, M, (int)p.P, np, BH, s);
        }
        const dim3 cg(np, BH);
        // the row statistics: from the forward's output and row records (denominators,
        // query offsets; dden from Y), made by the dQ kernel itself where it has the room,
        // else by a pass of their own; without them, a pass that recomputes each slice's
        // forward
        if (!Y)
            SLIM_TIMED("stats", s, kt->stats(cg, s, a));
        else if (kt->rowstat)
            SLIM_TIMED("rowstat", s,
                       kt->rowstat(dim3(np * (unsigned)((p.c + ROWSTAT_ROWS - 1) / ROWSTAT_ROWS), BH), s, a));
        if (kt->gstate) {
            if (dt)
                SLIM_TIMED("bwdq_dw", s, dt->bwdq(cg, s, a));
            else
                SLIM_TIMED("bwdq", s, kt->bwdq(cg, s, a));
            SLIM_TIMED("gstate", s, kt->gstate(cg, s, a));
        } else {
            if (dt)
                SLIM_TIMED("bwdq_gstate_dw", s, dt->bwdq(cg, s, a));
            else
                SLIM_TIMED("bwdq_gstate", s, kt->bwdq(cg, s, a));
        }
        scan(2, a.gslots, gR, gS, D, M, (int)p.P, np, BH, s);
        if (dt) {
            SLIM_TIMED("bwdkv_dw", s, dt->bwdkv(cg, s, a));
            // dW partials of this window's rows, then their fixed-order sum into dW
            // (the first window processed, the last one, writes it; the others add)
            DwArgs da;
            da.P[0] = a.pq; da.P[1] = a.pk; da.X[0] = Q; da.X[1] = K;
            da.part = (float *)(base + p.part_off);
            da.L = d->L;
            da.r0 = (long long)a.n0 * p.c;
            da.prows = p.P * p.c;
            const long long wl = d->L - da.r0 < (long long)np * p.c ? d->L - da.r0 : (long long)np * p.c;
            da.wl = (int)wl;
            dw_split(p.BH, wl, &da.S, &da.rps);
            SLIM_TIMED("dw", s, dt->dw(dim3(da.S, BH, 2), s, da));
            const int parts = 2 * BH * da.S, n4 = M * D / 4;
            const f4 *src = (const f4 *)da.part;
            int rows = parts;
            prof::Scope ps("dw_sum", s);
            if (rows > 32) {
                f4 *mid = (f4 *)(base + p.part2_off);
                const int r2 = (rows + 31) / 32;
                hipLaunchKernelGGL(sum_rows_kernel, dim3((n4 + 255) / 256, r2), dim3(256), 0, s, src, rows, n4, 32,
                                   mid, 0);
                src = mid;
                rows = r2;
            }
            hipLaunchKernelGGL(sum_rows_kernel, dim3((n4 + 255) / 256, 1), dim3(256), 0, s, src, rows, n4, rows,
                               (f4 *)dW, wi != nwin - 1 ? 1 : 0);
        } else {
            SLIM_TIMED("bwdkv", s, kt->bwdkv(cg, s, a));
        }
    }
    if (dR_in) {
        narrow2(dR_in, gR, p.BH * D * M, dS_in, gS, p.BH * M, f64, s);
    }
    return hipGetLastError() == hipSuccess ? SLIM_OK : SLIM_ERR_HIP;
}

slim_status slim_decode_step(const slim_desc *d, const void *q, const void *k, const void *v, const void *W,
                             const void *R_in, const void *S_in, void *y, void *R_out, void *S_out, void *stream)
{
    slim_status st = slim_validate(d, SLIM_PASS_DECODE);
    if (st != SLIM_OK) return st;
    if (!q || !k || !v || !y || !R_out || !S_out) return SLIM_ERR_NULL;
    if (d->feat == SLIM_FEAT_FAVOR && !W) return SLIM_ERR_NULL;
    if (d->feat == SLIM_FEAT_ELU1 && W) return SLIM_ERR_SHAPE;
    if ((R_in == nullptr) != (S_in == nullptr)) return SLIM_ERR_NULL;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(W, 16) || misaligned(y, 16) ||
        misaligned(R_in, 16) || misaligned(S_in, 16) || misaligned(R_out, 16) || misaligned(S_out, 16))
        return SLIM_ERR_ALIGN;
    // the state may be updated in place, but not through partly overlapping ranges
    const long long BH = d->B * d->H;
    const bool f64 = d->state_dtype == SLIM_F64;
    const long long es = f64 ? 8 : 4;
    if (overlaps_partly(R_in, R_out, BH * d->d * d->M * es) || overlaps_partly(S_in, S_out, BH * d->M * es))
        return SLIM_ERR_SHAPE;
    const KernelTable *kt = find(d);
    hipStream_t s = (hipStream_t)stream;
    DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.W = W;
    a.Rin = R_in; a.Sin = S_in; a.y = y; a.Rout = R_out; a.Sout = S_out;
    SLIM_TIMED("decode", s, kt->decode(dim3((unsigned)(d->B * d->H)), s, a, f64));
    return hipGetLastError() == hipSuccess ? SLIM_OK : SLIM_ERR_HIP;
}

}  // extern "C"
