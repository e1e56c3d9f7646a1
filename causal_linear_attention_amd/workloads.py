"""The five synthetic workloads the attention path is checked and measured on.

Shapes follow the page's statement of the operation (Q, K, V in R^{B x H x L x d},
g: R^d -> R_+^M) with a user-chosen slice count; "chunks" is the number of
slices N and the slice (chunk) length is ceil(L / N).  Inputs are Gaussian as
listed; ``qkv_scale`` multiplies N(0, 1) draws of Q, K, V, and dY is N(0, 1).
Where a workload leaves a choice open (W draw, distribution) the plainest
reading is taken: W iid N(0, 1) unless "orthogonal" is named.
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    d: int
    M: int
    chunks: int          # number of slices N; slice length = ceil(L / N)
    dtype: str           # "f32" or "bf16": dtype of Q, K, V, W, dY, Y, dQ, dK, dV
    feat: str            # "favor" or "elu1"
    w_kind: str          # "gaussian" or "orthogonal" (FAVOR+ only)
    qkv_scale: float
    seed: int
    backward: bool = True

    @property
    def chunk_len(self) -> int:
        return -(-self.L // self.chunks)

    @property
    def tokens(self) -> int:
        return self.B * self.L

    @property
    def head_tokens(self) -> int:
        return self.B * self.H * self.L


WORKLOADS = {
    w.name: w
    for w in [
        # fp32 forward, L=256, d=M=16, four slices of 64, W ~ N(0,1), Q,K,V ~ N(0, 0.5^2)
        Workload("favor_f32_L256_d16_M16", 1, 1, 256, 16, 16, 4, "f32", "favor", "gaussian", 0.5, 1,
                 backward=False),
        # fp32 fwd+bwd, orthogonal random features, slices of 256
        Workload("favor_ortho_f32_L4096_d64_M128", 2, 8, 4096, 64, 128, 16, "f32", "favor",
                 "orthogonal", 64 ** -0.25, 2),
        # bf16 fwd+bwd, fp32 state/accumulation, slices of 512 (the headline measurement)
        Workload("favor_bf16_L16384_d64_M256", 4, 16, 16384, 64, 256, 32, "bf16", "favor", "gaussian",
                 64 ** -0.25, 3),
        # bf16 long context, 2048 slices of 512
        Workload("favor_bf16_L1048576_d64_M64", 1, 8, 1 << 20, 64, 64, 2048, "bf16", "favor",
                 "gaussian", 64 ** -0.25, 4),
        # bf16 elementwise elu(x)+1, M = d = 128, slices of 256
        Workload("elu1_bf16_L8192_d128", 8, 12, 8192, 128, 128, 32, "bf16", "elu1", "gaussian", 1.0, 5),
    ]
}

HEADLINE = "favor_bf16_L16384_d64_M256"


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """Recurrent decoding: every step feeds one new token to each of B sequences
    (all H heads) and updates their (d+1) x M fp32 states in place.  The state
    of each head starts as the state after a `prefix`-token prompt."""
    name: str
    B: int
    H: int
    d: int
    M: int
    dtype: str
    feat: str
    w_kind: str
    qkv_scale: float
    seed: int
    prefix: int = 64

    @property
    def heads(self) -> int:
        return self.B * self.H


DECODE_WORKLOADS = {
    w.name: w
    for w in [
        # the headline head shape, 512 sequences: 545 MB of state, more than the on-chip caches hold
        DecodeWorkload("decode_favor_bf16_B512_H16_d64_M256", 512, 16, 64, 256, "bf16", "favor", "gaussian",
                       64 ** -0.25, 6),
        # 32 sequences: 34 MB of state, small enough to stay in the last-level cache between steps
        DecodeWorkload("decode_favor_bf16_B32_H16_d64_M256", 32, 16, 64, 256, "bf16", "favor", "gaussian",
                       64 ** -0.25, 6),
    ]
}

DECODE_HEADLINE = "decode_favor_bf16_B512_H16_d64_M256"


def decode_bytes_per_head(w: DecodeWorkload) -> int:
    """Algorithmic HBM bytes of one decode step per head: the fp32 state [R; S]
    read and written once, q, k, v read and y written once (W, shared by all
    heads, is counted once per launch, not here)."""
    s = 2 if w.dtype == "bf16" else 4
    return 2 * (w.d + 1) * w.M * 4 + 4 * w.d * s


def io_bytes_per_head_token(w: Workload, backward: bool = True) -> float:
    """Minimum HBM traffic per (token, head): read Q, K, V (+ dY) and write Y
    (+ dQ, dK, dV) once, in the I/O dtype."""
    s = 4 if w.dtype == "f32" else 2
    n = 11 if backward else 4
    return n * w.d * s


def kernel_flops(w: Workload, tile: int) -> dict:
    """Useful MFMA floating-point work per (token, head) of each kernel, as the
    kernels evaluate it: every chunk is walked in `tile`-row tiles carrying the
    d x M state, so the intra-tile causal products cost about (tile+1) M and
    (tile+1) d per row, and every state-sized product (a d x M contraction per
    row) costs 2 d M.  A FAVOR+ feature-map projection is one more 2 d M per row
    and input it is applied to (elu+1 needs none).  Zero padding, masked-out
    upper triangles and elementwise work are not counted."""
    d, M = w.d, w.M
    favor = w.feat == "favor"
    P = 2 * d * M if favor else 0        # one feature-map projection
    dm = 2 * d * M                       # one state-sized contraction
    tm = (tile + 1) * M                  # causal tile x tile x M product, per row
    td = (tile + 1) * d                  # causal tile x tile x d product, per row
    vjp = dm if favor else 0             # FAVOR+ chain rule through W
    return {
        "state": P + dm,                                   # g(K); [R | S] += g(K)^T [V | 1]
        "fwd": 2 * P + tm + td + 2 * dm,                   # g(Q), g(K); P^T; [V | 1]^T P^T; R g(Q); state
        "stats": 2 * P + tm + td + 2 * dm,                 # the fwd tile (numerators dotted with dY); state
        "bwdq": 2 * P + tm + td + 2 * dm + vjp,            # g(Q), g(K); A^T; g(K)^T A^T; R^T dNum; W chain; R
        "gstate": P + dm,                                  # g(Q); dG += g(Q)^T [dNum | dden]
        "bwdq_gstate": 2 * P + tm + td + 3 * dm + vjp,     # bwdq, and dG += g(Q)^T [dNum | dden]
        "bwdkv": 2 * P + 2 * tm + 2 * td + 3 * dm + vjp,   # g(Q), g(K); P; dNum^T P; dR g(K)^T; A;
                                                            # g(Q)^T A; dR^T V; W chain; dR update
        # the dW pass: the same dQ and dK/dV work (they also store dg(X) . g(X)), and the
        # row contraction dW += (dg(X) . g(X))^T X for X = Q and K
        "bwdq_dw": 2 * P + tm + td + 2 * dm + vjp,
        "bwdq_gstate_dw": 2 * P + tm + td + 3 * dm + vjp,
        "bwdkv_dw": 2 * P + 2 * tm + 2 * td + 3 * dm + vjp,
        "dw": 2 * dm if favor else 0,
    }


def kernel_bytes(w: Workload, group: int = 1, fr: bool = False) -> dict:
    """Algorithmic HBM bytes per (token, head) of each chunk kernel and scan: every
    input tensor row read once, every output row written once, one (d+1) x M fp32
    state slot read or written per workgroup's group of `group` slices (so per row:
    slot / (group c)), 16 bytes of row statistics (1/den, dden, query offset, one
    unused float) per row where used.  fr: the dQ kernel makes the row statistics
    itself from the forward's output row and 8-byte row record (and stores them for
    the dK/dV kernel) instead of reading them.  No re-reads, no caches."""
    s = 2 if w.dtype == "bf16" else 4
    row = w.d * s                                   # one Q/K/V/Y/dY/dQ/dK/dV row
    slot = (w.d + 1) * w.M * 4 / min(w.chunk_len * group, w.L)  # one group's state, per row
    st = 16
    out = {
        "state": 2 * row + slot,                    # K, V -> chunk state
        "scan_prefix": 2 * slot, "scan_reverse": 2 * slot, "scan_grad": 2 * slot,  # slots in place
        "scan_window": 2 * slot, "scan_sum": slot,  # several windows: start states; the final-state sweep
        # Q, K, V, entry state -> Y, and (a step with a backward) 8 bytes of row statistics
        "fwd": 3 * row + slot + row + (8 if w.backward else 0),
        "stats": 4 * row + slot + st,               # Q, K, V, dY, entry state -> row statistics
        "rowstat": 2 * row + 8 + st,                # Y, dY, the forward's row statistics -> row statistics
        "bwdq": 4 * row + slot + st + row,          # Q, K, V, dY, entry state, statistics -> dQ
        "gstate": 2 * row + st + slot,              # Q, dY, statistics -> gradient slot
        "bwdq_gstate": 4 * row + 2 * slot + st + row,  # Q, K, V, dY, entry state, statistics -> dQ, gradient slot
        "bwdkv": 4 * row + st + slot + 2 * row,     # Q, K, V, dY, statistics, gradient slot -> dK, dV
        # the dW pass: each backward kernel also writes one row of dg(X) . g(X) (M operand-type
        # values), which the row contraction reads back with X (query and key side)
        "bwdq_dw": 4 * row + slot + st + row + w.M * s,
        "bwdq_gstate_dw": 4 * row + 2 * slot + st + row + w.M * s,
        "bwdkv_dw": 4 * row + st + slot + 2 * row + w.M * s,
        "dw": 2 * (w.M * s + row),
    }
    if fr:  # + the output row and the 8-byte record read, the statistics written, not read
        for k in ("bwdq", "bwdq_gstate", "bwdq_dw", "bwdq_gstate_dw"):
            out[k] += row + 8
    return out


def unsliced_flops(w: Workload) -> float:
    """The per-(token, head) fwd+bwd count of the unsliced-tile accounting:
    28 d M + 4 c (M + d) for FAVOR+, 16 d M + 4 c (M + d) for elu+1."""
    c = w.chunk_len
    base = 28 if w.feat == "favor" else 16
    return base * w.d * w.M + 4 * c * (w.M + w.d)
