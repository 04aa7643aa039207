"""fp8 (OCP e4m3) emulation of the softmax branch (oracle, test
infrastructure only).

The VDN-H3 article's performance section reports an fp8 version without
saying which operations are fp8.  The library's reading, which this module
writes out:

* the softmax branch's Q, K, V (video and text) are quantised per
  (tensor, batch, head) with scale s = absmax / 448, round-to-nearest-even
  and saturation; the scores are the exact products of the codes times the
  two scales;
* the probabilities that multiply V are rounded to e4m3 after scaling by
  2^8 (so that values down to 2^-17 stay representable), against a running
  row maximum taken per 64-key tile: the keys are walked frame by frame
  through S(f) in ascending frame order, each frame in tiles of 64 keys from
  its first token (the last tile of a frame may be short), then the text in
  tiles of 64; the running maximum m (log2 units) starts at -inf and moves to
  a tile's maximum only when that exceeds m by more than 0.75, so every
  scaled probability stays at most 2^8.75 < 448; when m moves, the sums
  gathered so far are multiplied by 2^(m_old - m_new);
* the normaliser sums the probabilities before their e4m3 rounding.

The result depends on the order of the walk (a probability's code depends on
the maximum seen up to its tile), which is why the walk is part of the
reading.  Decisions that pick a code or move the maximum are taken in
float32, as the kernel takes them: the scale s = float32(absmax) / 448,
x * (1 / s) in float32; the score of two code vectors rounded to float32,
times the float32 factor (s_q s_k) tau log2(e); the tile maximum compared
with m + 0.75 in float32; the scaled probability 2^(score + 8 - m) formed as
a float32 fused multiply-add followed by a float32 exp2.  Sums, the rescale
factors and the final division run in float64.

e4m3 (OCP FP8 E4M3): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
normal numbers 2^-6 .. 448, subnormals in steps of 2^-9, no infinities.

Pinned by tests/test_oracle_fp8.py: the rounding against torch's
float8_e4m3fn conversion and the format's closed forms; the branch by
uniform scores (the mean of the quantised values), inputs whose scaled
probabilities are all on the e4m3 grid (then equal to the unquantised
softmax branch on the dequantised inputs), unrounded probabilities against
the unquantised branch on random data, and hand-derived codes for a
frame-tiled walk, a maximum that rises inside a tile and a subnormal code;
planted mistakes in each step fail one of them.
"""
import math

import numpy as np

from .layout import frame_sets

E4M3_MAX = 448.0
KEY_TILE = 64          # keys per tile of the walk
P_SLACK = 0.75         # log2 units the running maximum may lag a tile maximum
P_SCALE_LOG2 = 8.0     # probabilities are rounded as P * 2^8
LOG2E = 1.4426950408889634


def round_e4m3(x):
    """Nearest e4m3 value (ties to even), saturated to +-448; float64 in/out."""
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # exponent of the binade, floored at the subnormal binade (2^-6)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    step = np.exp2(e - 3.0)            # 3 mantissa bits
    q = np.round(a / step) * step      # np.round: half to even
    return np.sign(x) * np.minimum(q, E4M3_MAX)


def quantise_codes(x, axes=(1, 3)):
    """Per-(batch, head) quantisation of a [B, tokens, H, D] tensor.
    Returns (e4m3 code values float64, scales float32 [B, H]); the
    dequantised tensor is codes * scale."""
    x32 = np.asarray(x, np.float32)
    if x32.shape[1] == 0:
        return np.zeros(x32.shape), np.ones((x32.shape[0], x32.shape[2]), np.float32)
    amax = np.max(np.abs(x32), axis=axes, keepdims=True)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    inv = (np.float32(1.0) / s).astype(np.float32)
    codes = round_e4m3((x32 * inv).astype(np.float32))
    return codes, s.reshape(s.shape[0], s.shape[2])


def quantise(x, axes=(1, 3)):
    """Per-(batch, head) quantisation of a [B, tokens, H, D] tensor.
    Returns (dequantised values float64, scales float32 [B, H])."""
    codes, s = quantise_codes(x, axes)
    return codes * s.astype(np.float64)[:, None, :, None], s


def scale_log2(D, scale=None):
    """float32 tau log2(e), tau = scale if given (> 0), else 1/sqrt(D) in
    float32."""
    tau = np.float32(scale) if scale else np.float32(1.0) / np.sqrt(np.float32(D))
    return np.float32(tau * np.float32(LOG2E))


def key_tiles(frames, n, L):
    """The walk: (segment, first key, key count) per tile; segment "v" is the
    video tensor (first key = token index), "t" the text."""
    out = []
    for g in sorted(frames):
        for t0 in range(0, n, KEY_TILE):
            out.append(("v", g * n + t0, min(KEY_TILE, n - t0)))
    for t0 in range(0, L, KEY_TILE):
        out.append(("t", t0, min(KEY_TILE, L - t0)))
    return out


def _exp2_f32(a32):
    return np.exp2(np.asarray(a32, np.float32)).astype(np.float32)


def ambiguous_step(p, rel):
    """For scaled probabilities p (0 <= p < 448) known to a relative accuracy
    rel: the distance between the two e4m3 values around p where p lies within
    rel * p of the rounding boundary between them, else 0."""
    p = np.asarray(p, np.float64)
    step = np.exp2(np.floor(np.log2(np.maximum(p, 2.0 ** -6))) - 3.0)
    mid = np.floor(p / step) * step + step / 2
    return np.where(np.abs(p - mid) <= rel * p, step, 0.0)


def online_rows(qc, tiles, round_p=True, mfma_prec=0.0, perturb=None):
    """Walk of one block of query rows.

    qc: [R, D] query codes.  tiles: list of (key codes [n_t, D], dequantised
    values [n_t, D] float64, float32 logit factor (s_q s_k) tau log2(e)).
    Returns ([R, D] float64, [R] margin, [R, D] bound or None).

    margin: the smallest |tile maximum - (m + slack)| over the row's
    decisions after the first (inf with one tile), less the error those
    decisions may carry under the model below: a row with margin <= 0 may
    decide otherwise on hardware and round its later probabilities against
    another maximum.

    mfma_prec > 0 gives a bound on how far hardware may land from this
    result when its matrix instruction returns each step of 64 products
    (64 consecutive head dimensions of a score, 64 keys of a tile for the
    probability-value product) only to within mfma_prec times the largest
    |product| of the step, its exp2 and fused multiply-add carry a float32
    ulp, and its float32 running sums one ulp per add.  Every scaled
    probability is then known to a relative accuracy rel; one within rel of
    an e4m3 rounding boundary may take the other code; a moved maximum
    rescales what was gathered by a factor known to the error of both
    maxima.  perturb (a numpy Generator) moves every score, probability and
    product step by a random amount inside that model -- the deviation the
    bound has to cover."""
    R, D = qc.shape
    m = np.full(R, -np.inf, np.float32)
    l = np.zeros(R)
    acc = np.zeros((R, D))
    margin = np.full(R, np.inf)
    slack = np.float32(P_SLACK)
    bound = np.zeros((R, D)) if mfma_prec else None
    mag = np.zeros((R, D))        # sum of |code| |value| gathered so far (units of the current maximum)
    em = np.zeros(R)              # error bound of the running maximum (log2 units)
    rmax = np.zeros(R)            # largest relative error of a probability or rescale in the row
    fp32_sums = len(tiles) * 2.0 ** -24
    steps = [slice(d0, min(D, d0 + 64)) for d0 in range(0, D, 64)]
    for kc, vd, dq in tiles:
        s32 = (qc @ kc.T).astype(np.float32)                        # exact sums, rounded once
        if mfma_prec:
            # largest |q_d k_d| of each 64-dimension step, bounded by max|q_d| max|k_d|
            big = sum(np.abs(qc[:, st]).max(axis=1)[:, None] * np.abs(kc[:, st]).max(axis=1)[None, :]
                      for st in steps)
            et = mfma_prec * big * float(dq)                        # error bound of each log2-score
            if perturb is not None:
                s32 = (s32 + mfma_prec * big * perturb.uniform(-1, 1, big.shape)).astype(np.float32)
        mx = (s32.max(axis=1) * dq).astype(np.float32)
        dec_err = 2.0 * et.max(axis=1) if mfma_prec else 0.0
        margin = np.minimum(margin, np.where(np.isneginf(m), np.inf, np.abs(mx - (m + slack)) - dec_err))
        grow = mx > m + slack
        m_new = np.where(grow, mx, m).astype(np.float32)
        alpha = np.where(grow, np.exp2(m.astype(np.float64) - m_new.astype(np.float64)), 1.0)
        alpha = np.where(np.isneginf(m), 0.0, alpha)
        acc *= alpha[:, None]
        l *= alpha
        m = m_new
        moff = (np.float32(P_SCALE_LOG2) - m).astype(np.float32)
        # fused multiply-add: s dq + moff is exact in float64, rounded once
        arg = (s32.astype(np.float64) * np.float64(dq) + moff.astype(np.float64)[:, None]).astype(np.float32)
        p = _exp2_f32(arg).astype(np.float64)                       # P * 2^8
        if perturb is not None:
            p = p * (1.0 + 2.0 ** -22 * perturb.uniform(-1, 1, p.shape))
        pw = round_e4m3(p) if round_p else p
        prod = pw @ vd
        if mfma_prec:
            mag_new = np.abs(pw) @ np.abs(vd)
            pv_err = mfma_prec * np.abs(pw).max(axis=1)[:, None] * np.abs(vd).max(axis=0)[None, :] \
                + fp32_sums * mag_new
            if perturb is not None:
                prod = prod + pv_err * perturb.uniform(-1, 1, prod.shape)
            em_new = np.where(grow, et.max(axis=1), em)
            ea = np.where(grow & (alpha > 0), np.log(2.0) * (em + em_new) + 2.0 ** -22, 0.0)
            em = em_new
            # one float32 ulp of the exponent argument (and of 8 - m) moves P by ln 2 ulp
            ulp = np.spacing(np.abs(arg)).astype(np.float64) + np.spacing(np.abs(moff)).astype(np.float64)[:, None]
            rel = np.log(2.0) * (et + em[:, None] + ulp) + 2.0 ** -21
            rmax = np.maximum(rmax, np.maximum(rel.max(axis=1), ea))
            bound = alpha[:, None] * (bound + ea[:, None] * mag)
            mag = alpha[:, None] * mag + mag_new
            bound += pv_err + (ambiguous_step(p, rel) @ np.abs(vd) if round_p else 0.0)
        acc += prod
        l += p.sum(axis=1)
    out = acc / l[:, None]
    if mfma_prec:
        bound = bound / l[:, None] + (rmax + fp32_sums)[:, None] * np.abs(out)
    return out, margin, bound


def softmax_branch_fp8(q, k, v, text_k, text_v, lay, scale=None, tokens=None, round_p=True, margins=False,
                       mfma_prec=0.0, perturb=None):
    """Softmax branch on the quantised inputs with the e4m3 probability
    rounding of the reading above; round_p=False keeps the probabilities
    unrounded (the quantisation of Q, K and V alone).  Returns
    [B, len(tokens), H, D] float64 (all video tokens when tokens is None);
    with margins=True also [B, len(tokens), H]: per row, how close (log2
    units) its closest decision on the running maximum came to going the
    other way (less its error under mfma_prec, see online_rows); with
    mfma_prec > 0 also the [B, len(tokens), H, D] deviation bound of
    online_rows.  perturb: see online_rows."""
    B, N, H, D = q.shape
    n, L = lay.tokens_per_frame, text_k.shape[1]
    sl2 = scale_log2(D, scale)
    qc, sq = quantise_codes(q)
    kc, sk = quantise_codes(k)
    vc, sv = quantise_codes(v)
    tkc, stk = quantise_codes(text_k)
    tvc, stv = quantise_codes(text_v)
    sets = frame_sets(lay.frames, lay.chunk_frames, lay.chunk_radius, lay.anchor_first, lay.anchor_last)
    rows = np.arange(N) if tokens is None else np.asarray(tokens)
    out = np.zeros((B, rows.size, H, D))
    marg = np.full((B, rows.size, H), np.inf)
    bnd = np.zeros((B, rows.size, H, D)) if mfma_prec else None
    frame_of = rows // n
    for f in range(lay.frames):
        sel = np.nonzero(frame_of == f)[0]
        if sel.size == 0:
            continue
        walk = key_tiles(sets[f][0], n, L)
        for b in range(B):
            for h in range(H):
                dqv = np.float32(np.float32(sq[b, h] * sk[b, h]) * sl2)
                dqt = np.float32(np.float32(sq[b, h] * stk[b, h]) * sl2)
                tiles = []
                for seg, t0, cnt in walk:
                    if seg == "v":
                        tiles.append((kc[b, t0:t0 + cnt, h], vc[b, t0:t0 + cnt, h] * np.float64(sv[b, h]), dqv))
                    else:
                        tiles.append((tkc[b, t0:t0 + cnt, h], tvc[b, t0:t0 + cnt, h] * np.float64(stv[b, h]),
                                      dqt))
                for s0 in range(0, sel.size, 512):
                    ii = sel[s0:s0 + 512]
                    o, mg, bd = online_rows(qc[b, rows[ii], h], tiles, round_p, mfma_prec, perturb)
                    out[b, ii, h], marg[b, ii, h] = o, mg
                    if mfma_prec:
                        bnd[b, ii, h] = bd
    if mfma_prec:
        return out, marg, bnd
    return (out, marg) if margins else out


def scales(inp):
    """float32 dequantisation scales [5, B, H] of q, k, v, text_k, text_v."""
    return np.stack([quantise_codes(inp[name])[1] for name in ("q", "k", "v", "text_k", "text_v")])
