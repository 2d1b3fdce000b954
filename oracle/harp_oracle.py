"""Plain fp64 CPU oracle for the HARP / randomized-Hadamard apply path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the C-ABI library
and its Python binding) imports, links or calls this module; only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` do.
It shares no code, table or constant generator with the HIP kernels.

Everything here is written for readability against the pages, not for speed:
numpy fp64, one stage at a time, a library matmul as the only primitive.

Sources (short tags used in the docstrings below):

  [TS]   "Technical Summary: HARP (Hadamard-Preconditioned Adaptive Rotation
         Processor)", gist.science, paper 2605.29843 (same text in the Chinese
         page of that site).  Sections: §2.1 Core Architecture, §2.2 Hadamard
         Preconditioning & Initialization, §2.4 Deployment Efficiency,
         §5 Significance and Claims.
  [ABS]  arXiv 2605.29843v1 abstract, "HARP: Hadamard-Preconditioned Adaptive
         Rotation Processor for Extreme LLM Quantization".
  [RHT]  arXiv 2605.06014 abstract, "Quantizing With Randomized Hadamard
         Transforms: Efficient Heuristic Now Proven".

Readings of points the pages leave open:

  R1  index digits: a row of length d is viewed as an array of shape
      (b_0, ..., b_{m-1}) in C order; stage t mixes digit t, so its stride is
      prod(b_{t+1:}).  [TS §2.1 "stride permutations"]
  R2  group c of stage t is the C-order linear index of the other digits.
  R3  product order: stage 0 acts first; forward M = S_{m-1} ... S_0 D_s.
  R4  the sign vector acts on the input (x -> s*x before stage 0).
  R5  a block acts as y_r = sum_k B[r, k] x_k.
  R6  Sylvester order is the natural (not sequency) order, scaled 1/sqrt(b).
  R7  QR fallback: Q of the QR factorisation of a caller-supplied standard
      normal b x b matrix, column signs fixed so that diag(R) > 0.
  R8  Cayley map Q = (I - A)(I + A)^-1 with A skew-symmetric, its strict
      upper triangle filled row-major from the group's parameters.
  R9  Givens rotation [[cos t, -sin t], [sin t, cos t]].
  R10 one parameter set per (stage, group).
  R11 int8 parameter storage: one fp32 scale per stage, symmetric, round to
      nearest even, codes in [-127, 127].
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "is_pow2", "sylvester", "qr_fallback", "mgs_qr", "givens", "cayley",
    "theta_counts", "gauss_stage_list", "materialize_blocks",
    "theta_groups", "quantize_theta", "dequantize_theta",
    "apply", "apply_inverse", "apply_vjp", "theta_vjp", "dense_operator", "fwht", "rht_compose",
    "rotate_weight", "round_bf16", "round_f32", "quantize_i8", "stored_blocks",
    "row_rel_l2",
]


# --------------------------------------------------------------------------
# base mixers and learnable orthogonal factors
# --------------------------------------------------------------------------

def is_pow2(b: int) -> bool:
    return b >= 1 and (b & (b - 1)) == 0


def sylvester(b: int) -> np.ndarray:
    """Normalised Sylvester Hadamard matrix of order b (a power of two).

    [TS §2.2] names the normalised Sylvester Hadamard as the fixed base mixer
    for power-of-two radices.  Reading R6: natural order, entry (r, k) is
    (-1)^popcount(r & k) / sqrt(b).
    """
    if not is_pow2(b):
        raise ValueError(f"Sylvester order must be a power of two, got {b}")
    r = np.arange(b)[:, None]
    k = np.arange(b)[None, :]
    parity = np.vectorize(lambda v: bin(int(v)).count("1") & 1)(r & k)
    return np.where(parity == 1, -1.0, 1.0) / np.sqrt(b)


def qr_fallback(z: np.ndarray) -> np.ndarray:
    """Deterministic orthogonal base mixer for a non-power-of-two radix.

    [TS §2.1, §2.2]: the Q factor of a QR factorisation of a fixed Gaussian
    matrix.  Reading R7: the sign of each column is chosen so that the
    triangular factor has a positive diagonal (this makes Q unique).
    """
    z = np.asarray(z, dtype=np.float64)
    q, r = np.linalg.qr(z)
    d = np.sign(np.diag(r))
    d[d == 0] = 1.0
    return q * d[None, :]


def mgs_qr(z: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Modified Gram-Schmidt QR with positive diagonal R (a second, textbook
    route to the same unique factorisation; used only to pin qr_fallback)."""
    z = np.asarray(z, dtype=np.float64)
    n = z.shape[1]
    q = z.copy()
    r = np.zeros((n, n))
    for j in range(n):
        for i in range(j):
            r[i, j] = q[:, i] @ q[:, j]
            q[:, j] = q[:, j] - r[i, j] * q[:, i]
        r[j, j] = np.sqrt(q[:, j] @ q[:, j])
        q[:, j] = q[:, j] / r[j, j]
    return q, r


def givens(theta: float) -> np.ndarray:
    """2 x 2 Givens rotation, the learnable factor for radix 2 [TS §2.2].
    Reading R9 for the sign convention."""
    c, s = np.cos(theta), np.sin(theta)
    return np.array([[c, -s], [s, c]])


def skew_from_params(params: np.ndarray, b: int) -> np.ndarray:
    """Skew-symmetric A whose strict upper triangle is filled row-major."""
    a = np.zeros((b, b))
    iu = np.triu_indices(b, k=1)
    a[iu] = np.asarray(params, dtype=np.float64)
    return a - a.T


def cayley(params: np.ndarray, b: int) -> np.ndarray:
    """Cayley map of a skew-symmetric matrix, the learnable factor for radix
    b > 2 [TS §2.2].  Reading R8: Q = (I - A)(I + A)^-1.  (I - A) and
    (I + A)^-1 commute, so Q is obtained as the solution of (I + A) Q = I - A.
    """
    a = skew_from_params(params, b)
    eye = np.eye(b)
    return np.linalg.solve(eye + a, eye - a)


# --------------------------------------------------------------------------
# parameter layout and block materialisation
# --------------------------------------------------------------------------

def theta_counts(schedule, d: int) -> list[int]:
    """Learnable parameters per stage: one angle per group for radix 2, and
    b(b-1)/2 skew entries per group otherwise (reading R10)."""
    out = []
    for b in schedule:
        per = 1 if b == 2 else b * (b - 1) // 2
        out.append((d // b) * per)
    return out


def gauss_stage_list(schedule) -> list[int]:
    """Stages whose radix is not a power of two: each takes one b x b
    Gaussian matrix for its QR base mixer, in stage order."""
    return [t for t, b in enumerate(schedule) if not is_pow2(b)]


def _check_schedule(schedule, d):
    if int(np.prod(schedule)) != d:
        raise ValueError(f"prod(schedule)={int(np.prod(schedule))} != d={d}")


def materialize_blocks(schedule, d: int, theta: np.ndarray, gauss: np.ndarray | None):
    """B_{t,c} = Q_{t,c}(theta) G_{b_t} for every stage t and group c [TS §2.2].

    theta: concatenation over stages of the per-group parameters (theta_counts).
    gauss: concatenation, over the stages listed by gauss_stage_list, of one
           b_t x b_t standard-normal matrix each (row-major).
    Returns a list over stages of arrays shaped (d / b_t, b_t, b_t).
    """
    _check_schedule(schedule, d)
    theta = np.asarray(theta, dtype=np.float64).ravel()
    gauss = np.zeros(0) if gauss is None else np.asarray(gauss, dtype=np.float64).ravel()
    counts = theta_counts(schedule, d)
    if theta.size != sum(counts):
        raise ValueError("theta has the wrong length")
    blocks = []
    tpos = 0
    gpos = 0
    for t, b in enumerate(schedule):
        if is_pow2(b):
            g = sylvester(b)
        else:
            g = qr_fallback(gauss[gpos:gpos + b * b].reshape(b, b))
            gpos += b * b
        ngroups = d // b
        per = 1 if b == 2 else b * (b - 1) // 2
        th = theta[tpos:tpos + ngroups * per].reshape(ngroups, per)
        tpos += ngroups * per
        bt = np.empty((ngroups, b, b))
        for c in range(ngroups):
            q = givens(th[c, 0]) if b == 2 else cayley(th[c], b)
            bt[c] = q @ g
        blocks.append(bt)
    if gpos != gauss.size:
        raise ValueError("gauss has the wrong length")
    return blocks


def theta_groups(schedule, d: int) -> list[tuple[int, int]]:
    """(number of groups, parameters per group) for every stage: one angle per
    group for radix 2, b(b-1)/2 skew entries per group otherwise."""
    return [(d // b, 1 if b == 2 else b * (b - 1) // 2) for b in schedule]


def quantize_theta(schedule, d: int, theta: np.ndarray):
    """Symmetric int8 storage of the learnable parameters [TS §2.4: the
    parameters may be kept in int8].  Reading R11: one fp32 scale per stage,
    shared by all of that stage's parameters; scale = fp32(max|theta_stage| /
    127), code = clip(rint(theta / scale), -127, 127) with the decision taken
    in fp64; a stage of zeros gets scale 0 and codes 0.
    Returns (codes int8 of theta's length, scales fp32, one per stage)."""
    _check_schedule(schedule, d)
    theta = np.asarray(theta, dtype=np.float64).ravel()
    codes, scales = [], []
    pos = 0
    for ng, per in theta_groups(schedule, d):
        th = theta[pos:pos + ng * per]
        pos += ng * per
        amax = np.abs(th).max() if th.size else 0.0
        scale = float(np.float32(amax / 127.0))
        if scale > 0:
            code = np.clip(np.rint(th / scale), -127, 127)
        else:
            code = np.zeros_like(th)
        codes.append(code.astype(np.int8))
        scales.append(scale)
    if pos != theta.size:
        raise ValueError("theta has the wrong length")
    return np.concatenate(codes), np.array(scales, dtype=np.float32)


def dequantize_theta(schedule, d: int, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """theta = code * scale for every parameter, with its stage's scale
    (reading R11).  The product of an int8 and an fp32 is exact in fp64."""
    _check_schedule(schedule, d)
    codes = np.asarray(codes).ravel().astype(np.float64)
    scales = np.asarray(scales, dtype=np.float32).ravel().astype(np.float64)
    if scales.size != len(schedule):
        raise ValueError("one scale per stage expected")
    out = []
    pos = 0
    for t, (ng, per) in enumerate(theta_groups(schedule, d)):
        out.append(codes[pos:pos + ng * per] * scales[t])
        pos += ng * per
    if pos != codes.size:
        raise ValueError("codes have the wrong length")
    return np.concatenate(out)


# --------------------------------------------------------------------------
# the structured transform
# --------------------------------------------------------------------------

def _stage(x: np.ndarray, schedule, t: int, bt: np.ndarray, transpose: bool) -> np.ndarray:
    """One stage: the block of group c acts along digit t [TS §2.1, §2.2].

    x has shape (rows, d).  The row is viewed as (b_0, ..., b_{m-1}); digit t
    is moved last, the other digits (C order) index the group (R1, R2).
    """
    rows = x.shape[0]
    m = len(schedule)
    b = schedule[t]
    v = x.reshape((rows,) + tuple(schedule))
    v = np.moveaxis(v, 1 + t, m)                  # (rows, other digits..., b)
    other_shape = v.shape[1:m]
    v = v.reshape(rows, -1, b)                    # (rows, groups, b)
    mat = np.transpose(bt, (0, 2, 1)) if transpose else bt
    # y[n, c, r] = sum_k mat[c, r, k] v[n, c, k]   (reading R5)
    y = np.matmul(mat[None, :, :, :], v[:, :, :, None])[..., 0]
    y = y.reshape((rows,) + other_shape + (b,))
    y = np.moveaxis(y, m, 1 + t)
    return y.reshape(rows, -1)


def apply(x: np.ndarray, schedule, blocks, signs=None) -> np.ndarray:
    """Forward transform y = S_{m-1} ... S_0 D_s x for every row of x.

    [TS §2.1]: a product of block-diagonal stages over a mixed-radix schedule;
    readings R3 (order) and R4 (sign on the input).
    """
    x = np.asarray(x, dtype=np.float64)
    squeeze = x.ndim == 1
    x = np.atleast_2d(x)
    d = x.shape[1]
    _check_schedule(schedule, d)
    if signs is not None:
        x = x * np.asarray(signs, dtype=np.float64)[None, :]
    for t in range(len(schedule)):
        x = _stage(x, schedule, t, blocks[t], transpose=False)
    return x[0] if squeeze else x


def apply_inverse(y: np.ndarray, schedule, blocks, signs=None) -> np.ndarray:
    """Inverse x = D_s S_0^T ... S_{m-1}^T y: transposed blocks in reverse
    stage order, then the sign.  Exact because every block is orthogonal, so
    the processor is an exact change of basis [TS §2.1, §5; ABS]."""
    y = np.asarray(y, dtype=np.float64)
    squeeze = y.ndim == 1
    y = np.atleast_2d(y)
    d = y.shape[1]
    _check_schedule(schedule, d)
    for t in reversed(range(len(schedule))):
        y = _stage(y, schedule, t, blocks[t], transpose=True)
    if signs is not None:
        y = y * np.asarray(signs, dtype=np.float64)[None, :]
    return y[0] if squeeze else y


def _groups(x: np.ndarray, schedule, t: int) -> np.ndarray:
    """(rows, groups, b_t) copy of x: digit t last, group c the C-order index of
    the other digits (readings R1, R2)."""
    rows = x.shape[0]
    m = len(schedule)
    v = np.moveaxis(x.reshape((rows,) + tuple(schedule)), 1 + t, m)
    return v.reshape(rows, -1, schedule[t])


def apply_vjp(x: np.ndarray, schedule, blocks, signs, dy: np.ndarray):
    """Reverse-mode derivative of the forward transform against an upstream
    gradient dy (one per row), for fitting Theta by gradient descent on a
    calibration loss [TS §2.3].  For L = sum over rows of <dy, y>,
    y = S_{m-1} ... S_0 D_s x:

      x_0 = D_s x, x_{t+1} = S_t x_t;  g_m = dy, g_t = S_t^T g_{t+1};
      dL/dB_{t,c}[r, k] = sum over rows of g_{t+1}[c, r] x_t[c, k];
      dL/dx = D_s g_0.

    Returns (dx, dblocks) with dblocks[t] shaped like blocks[t]."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    dy = np.atleast_2d(np.asarray(dy, dtype=np.float64))
    d = x.shape[1]
    _check_schedule(schedule, d)
    s = np.ones(d) if signs is None else np.asarray(signs, dtype=np.float64)
    acts = []
    v = x * s[None, :]
    for t in range(len(schedule)):
        acts.append(v)
        v = _stage(v, schedule, t, blocks[t], transpose=False)
    g = dy
    dblocks = [None] * len(schedule)
    for t in reversed(range(len(schedule))):
        gv = _groups(g, schedule, t)
        xv = _groups(acts[t], schedule, t)
        dblocks[t] = np.einsum("ncr,nck->crk", gv, xv)
        g = _stage(g, schedule, t, blocks[t], transpose=True)
    return g * s[None, :], dblocks


def theta_vjp(schedule, d: int, theta: np.ndarray, gauss: np.ndarray | None, dblocks):
    """Chain dL/dB_{t,c} back to the parameters through B = Q(theta) G
    [TS §2.2]: dL/dQ = dL/dB G^T, then

      Givens (R9):  dQ/dtheta = [[-sin, -cos], [cos, -sin]];
      Cayley (R8):  Q = (I - A) M with M = (I + A)^-1, so
                    dQ = -(I + Q) dA M and dL/dA = -(I + Q)^T (dL/dQ) M^T;
                    A is U - U^T with U's strict upper triangle the group's
                    parameters (row-major), so dL/dtheta_(r,k) = dL/dA[r,k] - dL/dA[k,r].

    Returns dtheta in theta's layout."""
    _check_schedule(schedule, d)
    theta = np.asarray(theta, dtype=np.float64).ravel()
    gauss = np.zeros(0) if gauss is None else np.asarray(gauss, dtype=np.float64).ravel()
    out = np.zeros_like(theta)
    tpos = gpos = 0
    for t, b in enumerate(schedule):
        if is_pow2(b):
            g = sylvester(b)
        else:
            g = qr_fallback(gauss[gpos:gpos + b * b].reshape(b, b))
            gpos += b * b
        ngroups = d // b
        per = 1 if b == 2 else b * (b - 1) // 2
        iu = np.triu_indices(b, k=1)
        for c in range(ngroups):
            gq = np.asarray(dblocks[t][c], dtype=np.float64) @ g.T
            th = theta[tpos + c * per: tpos + (c + 1) * per]
            if b == 2:
                cs, sn = np.cos(th[0]), np.sin(th[0])
                out[tpos + c] = np.sum(gq * np.array([[-sn, -cs], [cs, -sn]]))
            else:
                a = skew_from_params(th, b)
                eye = np.eye(b)
                minv = np.linalg.inv(eye + a)
                q = (eye - a) @ minv
                da = -(eye + q).T @ gq @ minv.T
                out[tpos + c * per: tpos + (c + 1) * per] = da[iu] - da.T[iu]
        tpos += ngroups * per
    return out


def dense_operator(schedule, blocks, signs=None) -> np.ndarray:
    """The d x d matrix M with M e_j = apply(e_j) (column j)."""
    d = int(np.prod(schedule))
    return apply(np.eye(d), schedule, blocks, signs).T


# --------------------------------------------------------------------------
# randomized Hadamard transforms
# --------------------------------------------------------------------------

def fwht(x: np.ndarray) -> np.ndarray:
    """Normalised fast Walsh-Hadamard transform along the last axis, natural
    (Sylvester) order: the textbook in-place butterfly, then 1/sqrt(d)."""
    x = np.array(x, dtype=np.float64, copy=True)
    d = x.shape[-1]
    if not is_pow2(d):
        raise ValueError("fwht needs a power-of-two length")
    h = 1
    while h < d:
        v = x.reshape(x.shape[:-1] + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        x = v.reshape(x.shape)
        h *= 2
    return x / np.sqrt(d)


def rht_compose(x: np.ndarray, signs: np.ndarray, inverse: bool = False) -> np.ndarray:
    """k composed randomized Hadamard transforms, y = H D_k ... H D_1 x.

    [RHT] composes two or three independent RHTs (sign vector, then a
    normalised Hadamard); signs has shape (k, d).  The inverse is
    D_1 H ... D_k H y because H is symmetric and orthogonal.
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    signs = np.atleast_2d(np.asarray(signs, dtype=np.float64))
    if not inverse:
        for s in signs:
            x = fwht(x * s[None, :])
    else:
        for s in signs[::-1]:
            x = fwht(x) * s[None, :]
    return x


def rotate_weight(w: np.ndarray, su, blocks_u, signs_u, sv, blocks_v, signs_v,
                  inverse: bool = False) -> np.ndarray:
    """Two-sided processor on a weight matrix W (d_out x d_in).

    [TS §2, §3; ABS]: HARP is two-sided: an output-side rotation U and an
    input-side rotation V.  Forward W~ = M_U W M_V^T (M_V on every row, M_U on
    every column); inverse W = M_U^T W~ M_V.
    """
    w = np.asarray(w, dtype=np.float64)
    if not inverse:
        rows = apply(w, sv, blocks_v, signs_v)             # W M_V^T
        return apply(rows.T, su, blocks_u, signs_u).T      # M_U (.)
    rows = apply_inverse(w, sv, blocks_v, signs_v)         # W M_V
    return apply_inverse(rows.T, su, blocks_u, signs_u).T  # M_U^T (.)


# --------------------------------------------------------------------------
# stored (rounded) block values: the oracle rounds its own fp64 blocks
# --------------------------------------------------------------------------

def round_f32(v):
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(v):
    """Round fp64 values to the nearest bfloat16 (8 significant bits), ties to
    even, directly from fp64 (no intermediate fp32 rounding).  Normal range
    only; zero maps to zero."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                 # v = m 2^e, 0.5 <= |m| < 1
    q = np.rint(m * 256.0)             # np.rint rounds half to even
    out = np.ldexp(q, e - 8)
    tiny = (v != 0) & (np.abs(v) < 2.0 ** -126)
    if np.any(tiny):
        raise ValueError("round_bf16: subnormal bfloat16 range not modelled")
    return out


def quantize_i8(bt: np.ndarray):
    """Symmetric int8 storage of a stage's blocks with one fp32 scale per
    block ([TS §2.4] stores parameters in int8; this applies the same idea to
    the materialised blocks).  scale = fp32(max|B| / 127); code =
    clip(rint(B / scale), -127, 127), the decision taken in fp64."""
    bt = np.asarray(bt, dtype=np.float64)
    amax = np.abs(bt).reshape(bt.shape[0], -1).max(axis=1)
    scale = (amax / 127.0).astype(np.float32).astype(np.float64)
    scale_safe = np.where(scale > 0, scale, 1.0)
    code = np.clip(np.rint(bt / scale_safe[:, None, None]), -127, 127)
    code = np.where(scale[:, None, None] > 0, code, 0.0)
    return code.astype(np.int8), scale.astype(np.float32)


def stored_blocks(blocks, dtype: str):
    """The block values a kernel actually multiplies by, for each storage
    format: 'f64' (exact), 'f32', 'bf16', 'i8' (code * scale) and 'bf16x2'
    (hi + lo, hi = bf16(B), lo = bf16(B - hi))."""
    out = []
    for bt in blocks:
        if dtype == "f64":
            out.append(np.asarray(bt, dtype=np.float64))
        elif dtype == "f32":
            out.append(round_f32(bt))
        elif dtype == "bf16":
            out.append(round_bf16(bt))
        elif dtype == "i8":
            code, scale = quantize_i8(bt)
            out.append(code.astype(np.float64) * scale.astype(np.float64)[:, None, None])
        elif dtype == "bf16x2":
            hi = round_bf16(bt)
            lo = round_bf16(np.asarray(bt, dtype=np.float64) - hi)
            out.append(hi + lo)
        else:
            raise ValueError(dtype)
    return out


# --------------------------------------------------------------------------
# error metric
# --------------------------------------------------------------------------

def row_rel_l2(y: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row relative l2 error ||y - ref|| / ||ref|| (absolute l2 for a zero
    reference row)."""
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    ref = np.atleast_2d(np.asarray(ref, dtype=np.float64))
    num = np.linalg.norm(y - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
