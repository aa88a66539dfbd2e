"""fp64 numpy forwards of the collection's networks, with the probabilistic
rounding bound of an fp32 evaluation (test infrastructure).

Written from the shapes the pages give ("PPO CUDA Pipeline Design", Kernel
Phases, Phase A steps 3, 5 and 9; "GPU Pipeline Phase 2b", Kernel Components
1 and 2); used by the oracle's network pins and by the bf16 parity gate.
Each layer returns its fp64 output and a variance proxy: the sum of squared
bounds of the independent roundings that reach it (Higham and Mary, "A New
Approach to Probabilistic Rounding Error Analysis", SIAM J. Sci. Comput.
41(5), 2019); LAMBDA * sqrt(var) bounds an fp32 evaluation's distance from
the fp64 value except with probability 2 exp(-LAMBDA^2 / 2).
"""
import numpy as np

U = 2.0 ** -24
LAMBDA = 8.0


def bf16(x):
    """Round to the nearest bfloat16 (ties to even), returned as float64."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def dense(W, b, x, var, relu, bf=False):
    """One [out, in] layer on a batch of rows x [R, in] whose entries carry
    error variance proxies var.  Returns (y, var) in fp64."""
    W64 = np.asarray(W, np.float64)
    if bf:
        W64 = bf16(W)
        # an input known exactly (var == 0, the stored state) rounds the same
        # on both sides; one with an error may land on the neighbouring value
        var = np.where(var > 0, var + (2.0 ** -7 * np.abs(x)) ** 2, 0.0)
        x = bf16(x)
    b64 = np.asarray(b, np.float64)
    y = x @ W64.T + b64
    k = W64.shape[1]
    absum = np.abs(x) @ np.abs(W64).T + np.abs(b64)
    var = var @ (W64 * W64).T + (2 * k + 2) * U * U * absum * absum
    if relu:
        y = np.maximum(y, 0.0)
    return y, var


def mlp(ws, x, relu_mask, bf=False):
    """Chain of layers: ws = [W1, b1, W2, b2, ...]; relu_mask[l] says whether
    layer l is followed by ReLU."""
    return _chain(ws, x, np.zeros_like(x), relu_mask, bf)


def _chain(ws, x, var, relu_mask, bf=False):
    for l in range(len(ws) // 2):
        x, var = dense(ws[2 * l], ws[2 * l + 1], x, var, relu_mask[l], bf)
    return x, var


ACTOR_RELU = (True, True, False)
CRITIC_RELU = (True, True, True, True, True, False)
CURIOSITY_RELU = (True, False)


def dueling(ws, s, trunk_relu=(True, True), head_relu=(True, True)):
    """Q of a dueling net on rows s and its variance proxy; ws = [trunk 1,
    trunk 2, value 1, value 2, advantage 1, advantage 2] as (W, b) pairs."""
    h, vh = mlp(ws[0:4], s, trunk_relu)
    v, vv = _chain(ws[4:8], h, vh, (head_relu[0], False))
    a, va = _chain(ws[8:12], h, vh, (head_relu[1], False))
    mean = a.sum(axis=1, keepdims=True) / 45.0
    vmean = (va.sum(axis=1, keepdims=True)
             + 92 * U * U * np.abs(a).sum(axis=1, keepdims=True) ** 2) / 45.0 ** 2
    q = v + (a - mean)
    # (x + y + z)^2 <= 3 (x^2 + y^2 + z^2): the three parts are correlated
    vq = 3 * (vv + va + vmean) + 3 * U * U * (np.abs(v) + np.abs(a) + np.abs(mean)) ** 2
    return q, vq


def forward_inputs(ws, x, relu_mask, bf=True):
    """The input of every layer (bf16-rounded in the bf16 mode) and the
    output, fp64, for rows x."""
    ins = []
    for l in range(len(ws) // 2):
        W = bf16(ws[2 * l]) if bf else np.asarray(ws[2 * l], np.float64)
        xin = bf16(x) if bf else x
        ins.append(xin)
        x = xin @ W.T + np.asarray(ws[2 * l + 1], np.float64)
        if relu_mask[l]:
            x = np.maximum(x, 0.0)
    return ins, x


def _bf16_neighbour(v, up):
    """The next larger (up) or smaller bfloat16 value of a positive bf16 v."""
    b = np.asarray(v, np.float32).view(np.uint32).astype(np.int64)
    b = b + (1 << 16) if up else b - (1 << 16)
    return np.asarray([b], np.int64).astype(np.uint32).view(np.float32).astype(np.float64)[0]


def flip_effects(ws, x, relu_mask, rng):
    """For each row of x: the change of every output of the bf16 forward when
    one nonzero hidden-layer input (the input of a layer after the first),
    chosen at random, moves to a neighbouring bf16 value -- the effect of one
    rounding decision taken the other way.  Returns [rows, out] fp64."""
    ins, y = forward_inputs(ws, x, relu_mask)
    nl = len(ws) // 2
    out = np.zeros_like(y)
    for r in range(x.shape[0]):
        cand = [(l, i) for l in range(1, nl) for i in np.nonzero(ins[l][r])[0]]
        if not cand:
            continue
        l, i = cand[rng.integers(len(cand))]
        z = ins[l][r].copy()
        z[i] = _bf16_neighbour(z[i], bool(rng.integers(2)))
        for m in range(l, nl):
            zin = z if m == l else bf16(z)
            z = zin @ bf16(ws[2 * m]).T + np.asarray(ws[2 * m + 1], np.float64)
            if relu_mask[m]:
                z = np.maximum(z, 0.0)
        out[r] = np.abs(z - y[r])
    return out
