"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError if
the oracle disagrees with:
  * a closed form or special case the pages fix
      - zero offsets + zero mask logits -> 3x3 zero-padded box average
        (wmrh.cn/news/61976, the "细节亮点" note on zero-initialised offset and
        mask: the operator then acts as an ordinary 3x3 convolution);
      - offsets whose scaled value is an integer -> an exact gather;
      - constant input with softmax weights -> the constant (partition of unity);
      - samples far outside the map -> exactly zero (zero padding);
  * a library routine that computes the same thing another way
      - torch.nn.functional.grid_sample (bilinear, zeros, align_corners=False),
        the routine the pages' pure-PyTorch fallback is built on
        (wmrh.cn/news/61976 section 二 step 4), with torch autograd for the
        backward;
      - torch.nn.functional.conv2d (depthwise) for the point order, stride,
        dilation and padding conventions; avg_pool2d for the box average;
  * structural invariants: linearity in x and in the DCNv4 mask, shift
    invariance of the DCNv3 logits, group independence, the adjoint identity
    <F(x), g> = <x, F^T g>, central finite differences, and the softmax
    gradient summing to zero over the points;
  * hand-worked values in tests/golden/hand_bilinear.json;
  * a scalar loop per output element on tiny shapes (brute force).
They are written so that a plausible slip anywhere in the oracle (a dropped
term, a swapped (x, y) pair, a transposed point order, a wrong sign, a missing
offset_scale or softmax Jacobian) fails at least one of them;
tests/test_oracle_mutants.py checks exactly that on deliberately broken copies.
"""
from __future__ import annotations

import json
import pathlib

import numpy as np
import scipy.special
import torch
import torch.nn.functional as F

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden"


def _kw(groups, kernel=(3, 3), stride=(1, 1), pad=(1, 1), dilation=(1, 1), s=2.0, softmax=True,
        rc=False):
    kw = dict(groups=groups, kernel=kernel, stride=stride, pad=pad, dilation=dilation,
              offset_scale=s, softmax=softmax)
    if rc:
        kw["remove_center"] = True
    return kw


def _points(kernel, rc=False):
    """Grid positions (i, j) of the sampling points in order: row-major over
    the kernel, without the centre when it is removed."""
    pts = [(i, j) for i in range(kernel[0]) for j in range(kernel[1])]
    if rc:
        pts.remove((kernel[0] // 2, kernel[1] // 2))
    return pts


def _out(h, k, st, p, d):
    return (h + 2 * p - d * (k - 1) - 1) // st + 1


def _random_case(rng, n, h, w, c, g, kernel=(3, 3), stride=(1, 1), pad=(1, 1), dilation=(1, 1),
                 off_std=1.5, rc=False):
    ho = _out(h, kernel[0], stride[0], pad[0], dilation[0])
    wo = _out(w, kernel[1], stride[1], pad[1], dilation[1])
    K = len(_points(kernel, rc))
    x = rng.standard_normal((n, h, w, c))
    off = rng.standard_normal((n, ho, wo, g, K, 2)) * off_std
    m = rng.standard_normal((n, ho, wo, g, K))
    return x, off, m


def _close(a, b, tol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------- closed forms

def pin_box_average(orc):
    """Zero offsets and zero logits: every point weighs 1/9 and samples the
    regular 3x3 grid, i.e. a zero-padded 3x3 box average per channel."""
    rng = np.random.default_rng(101)
    for (n, h, w, c, g) in [(2, 7, 9, 32, 2), (1, 5, 4, 16, 4), (1, 1, 1, 16, 1)]:
        x = rng.standard_normal((n, h, w, c))
        off = np.zeros((n, h, w, g, 9, 2))
        m = np.zeros((n, h, w, g, 9))
        y = orc.forward(x, off, m, **_kw(g))
        xt = torch.from_numpy(x).permute(0, 3, 1, 2)
        ref = F.avg_pool2d(xt, 3, stride=1, padding=1, count_include_pad=True)
        _close(y, ref.permute(0, 2, 3, 1).numpy(), 1e-14, "box average")


def _exact_gather(x, off, m, groups, kernel, stride, pad, dilation, s, softmax):
    """Sum_k m_k * Xz[py, px] by numpy fancy indexing, for integer s*offset."""
    n, h, w, c = x.shape
    cg = c // groups
    _, ho, wo, _, K, _ = off.shape
    d = s * off
    assert np.all(d == np.round(d)), "the exact-gather pin needs integer s*offset"
    d = d.astype(np.int64)
    marg = int(np.abs(d).max()) + max(kernel) * max(dilation) + max(pad) + 2
    xp = np.zeros((n, h + 2 * marg, w + 2 * marg, groups, cg))
    xp[:, marg:marg + h, marg:marg + w] = x.reshape(n, h, w, groups, cg)
    N, HO, WO, G, KK = np.meshgrid(np.arange(n), np.arange(ho), np.arange(wo), np.arange(groups),
                                   np.arange(K), indexing="ij")
    i, j = KK // kernel[1], KK % kernel[1]
    py = HO * stride[0] - pad[0] + i * dilation[0] + d[..., 1]
    px = WO * stride[1] - pad[1] + j * dilation[1] + d[..., 0]
    vals = xp[N, py + marg, px + marg, G]                    # (n, ho, wo, G, K, cg)
    mk = scipy.special.softmax(m, axis=-1) if softmax else m
    y = (mk[..., None] * vals).sum(axis=4)                   # (n, ho, wo, G, cg)
    return y.reshape(n, ho, wo, c)


def pin_integer_offsets_exact_gather(orc):
    """Offsets with integer s*offset land on pixel centres: the bilinear sample
    is the pixel itself (or 0 outside), for any stride, pad, dilation."""
    rng = np.random.default_rng(102)
    cases = [
        dict(n=2, h=6, w=7, c=8, g=2, kernel=(3, 3), stride=(1, 1), pad=(1, 1), dilation=(1, 1), s=2.0),
        dict(n=1, h=9, w=8, c=6, g=3, kernel=(3, 3), stride=(2, 2), pad=(0, 1), dilation=(1, 2), s=2.0),
        dict(n=1, h=7, w=10, c=4, g=1, kernel=(3, 5), stride=(1, 2), pad=(2, 1), dilation=(2, 1), s=1.0),
        dict(n=1, h=5, w=5, c=3, g=3, kernel=(1, 1), stride=(1, 1), pad=(0, 0), dilation=(1, 1), s=0.5),
    ]
    for cs in cases:
        for softmax in (True, False):
            n, h, w, c, g = cs["n"], cs["h"], cs["w"], cs["c"], cs["g"]
            kernel, stride, pad, dil, s = cs["kernel"], cs["stride"], cs["pad"], cs["dilation"], cs["s"]
            ho = _out(h, kernel[0], stride[0], pad[0], dil[0])
            wo = _out(w, kernel[1], stride[1], pad[1], dil[1])
            K = kernel[0] * kernel[1]
            x = rng.standard_normal((n, h, w, c))
            off = rng.integers(-4, 5, size=(n, ho, wo, g, K, 2)) / s
            m = rng.standard_normal((n, ho, wo, g, K))
            y = orc.forward(x, off, m, **_kw(g, kernel, stride, pad, dil, s, softmax))
            ref = _exact_gather(x, off, m, g, kernel, stride, pad, dil, s, softmax)
            _close(y, ref, 1e-13, f"exact gather {cs} softmax={softmax}")


def pin_partition_of_unity(orc):
    """Constant input, softmax weights and every corner inside the map: the
    bilinear weights of each sample and the softmax weights each sum to 1, so
    the output equals the constant."""
    rng = np.random.default_rng(103)
    n, h, w, c, g, s = 2, 9, 11, 8, 2, 2.0
    x = np.full((n, h, w, c), 0.75)
    HO, WO = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
    K = 9
    kk = np.arange(K)
    i, j = kk // 3, kk % 3
    # target locations strictly inside [0, H-1) x [0, W-1)
    ty = rng.uniform(0.0, h - 1.0 - 1e-9, size=(n, h, w, g, K))
    tx = rng.uniform(0.0, w - 1.0 - 1e-9, size=(n, h, w, g, K))
    by = (HO[None, :, :, None, None] - 1 + i)
    bx = (WO[None, :, :, None, None] - 1 + j)
    off = np.stack([(tx - bx) / s, (ty - by) / s], axis=-1)
    m = rng.standard_normal((n, h, w, g, K))
    y = orc.forward(x, off, m, **_kw(g, s=s))
    _close(y, np.full_like(y, 0.75), 1e-13, "partition of unity")


def pin_out_of_range_is_zero(orc):
    """Samples beyond the map read zeros; infinite offsets put the sample
    outside; a NaN offset poisons only its own (pixel, group)."""
    rng = np.random.default_rng(104)
    n, h, w, c, g = 1, 6, 5, 8, 2
    x = rng.standard_normal((n, h, w, c))
    m = rng.standard_normal((n, h, w, g, 9))
    for big in (1e3, -1e3, np.inf, -np.inf, 1e300):
        off = np.full((n, h, w, g, 9, 2), big)
        y = orc.forward(x, off, m, **_kw(g))
        assert np.all(y == 0.0), f"offset {big} should give exact zeros"
    # only the y component far away: still outside
    off = rng.standard_normal((n, h, w, g, 9, 2))
    off[..., 1] = 50.0
    assert np.all(orc.forward(x, off, m, **_kw(g)) == 0.0)
    # one NaN offset in group 1 of pixel (2, 3)
    off = rng.standard_normal((n, h, w, g, 9, 2))
    off[0, 2, 3, 1, 4, 0] = np.nan
    y = orc.forward(x, off, m, **_kw(g))
    cg = c // g
    assert np.all(np.isnan(y[0, 2, 3, cg:])), "NaN offset must poison its group"
    y[0, 2, 3, cg:] = 0.0
    assert np.all(np.isfinite(y)), "NaN must not leak into other outputs"


def pin_hand_golden(orc):
    """Hand-worked values on a 2x2 map (tests/golden/hand_bilinear.json)."""
    d = json.loads((GOLDEN / "hand_bilinear.json").read_text())
    x = np.array(d["x"], dtype=np.float64)[None, :, :, None]   # (1, 2, 2, 1)
    for case in d["cases"]:
        ho, wo = case["pixel"]
        off = np.zeros((1, 2, 2, 1, 1, 2))
        off[0, ho, wo, 0, 0] = case["offset_xy"]
        m = np.ones((1, 2, 2, 1, 1))
        m[0, ho, wo, 0, 0] = case["mask"]
        y = orc.forward(x, off, m, **_kw(1, (1, 1), (1, 1), (0, 0), (1, 1), case["scale"], False))
        got = y[0, ho, wo, 0]
        assert abs(got - case["expected"]) < 1e-15, f"hand case {case}: got {got}"
    box = d["box_3x3_softmax"]
    y = orc.forward(x, np.zeros((1, 2, 2, 1, 9, 2)), np.zeros((1, 2, 2, 1, 9)), **_kw(1))
    _close(y[0, :, :, 0], np.array(box["expected"]), 1e-15, "hand box")


# --------------------------------------------------------------------------- invariants

def pin_linearity(orc):
    """F is linear in x (fixed offsets and mask); DCNv4 is linear in the mask;
    DCNv3 ignores a constant added to all logits of a (pixel, group)."""
    rng = np.random.default_rng(105)
    n, h, w, c, g = 2, 7, 6, 12, 3
    x, off, m = _random_case(rng, n, h, w, c, g)
    z = rng.standard_normal(x.shape)
    for softmax in (True, False):
        kw = _kw(g, softmax=softmax)
        lhs = orc.forward(2.5 * x - 0.75 * z, off, m, **kw)
        rhs = 2.5 * orc.forward(x, off, m, **kw) - 0.75 * orc.forward(z, off, m, **kw)
        _close(lhs, rhs, 1e-12, f"linearity in x (softmax={softmax})")
    m2 = rng.standard_normal(m.shape)
    kw = _kw(g, softmax=False)
    _close(orc.forward(x, off, m - 3.0 * m2, **kw),
           orc.forward(x, off, m, **kw) - 3.0 * orc.forward(x, off, m2, **kw),
           1e-12, "DCNv4 linearity in mask")
    shift = rng.standard_normal(m.shape[:-1])[..., None] * 4.0
    kw = _kw(g, softmax=True)
    _close(orc.forward(x, off, m + shift, **kw), orc.forward(x, off, m, **kw), 1e-12,
           "DCNv3 logit shift invariance")


def pin_group_independence(orc):
    """A G-group call equals G one-group calls on the groups' channel slices."""
    rng = np.random.default_rng(106)
    n, h, w, cg, g = 1, 6, 7, 5, 3
    x, off, m = _random_case(rng, n, h, w, cg * g, g)
    y = orc.forward(x, off, m, **_kw(g))
    for q in range(g):
        yq = orc.forward(x[..., q * cg:(q + 1) * cg], off[:, :, :, q:q + 1], m[:, :, :, q:q + 1],
                         **_kw(1))
        _close(y[..., q * cg:(q + 1) * cg], yq, 0.0, f"group {q}")


def pin_forward_pixels(orc):
    """The per-pixel entry point agrees with the whole-tensor one."""
    rng = np.random.default_rng(107)
    x, off, m = _random_case(rng, 2, 6, 5, 8, 2)
    y = orc.forward(x, off, m, **_kw(2))
    pix = np.array([0, 7, 29, 30, 59])
    yp = orc.forward_pixels(x, off, m, pix, **_kw(2))
    _close(yp, y.reshape(-1, 8)[pix], 0.0, "forward_pixels")


def pin_out_size(orc):
    """Output extent matches torch's convolution shape rule."""
    for (h, k, st, p, d) in [(96, 3, 1, 1, 1), (9, 3, 2, 0, 1), (10, 5, 2, 2, 2), (7, 3, 3, 1, 2),
                             (1, 1, 1, 0, 1), (5, 3, 1, 0, 2)]:
        t = F.conv2d(torch.zeros(1, 1, h, h), torch.zeros(1, 1, k, k), stride=st, padding=p,
                     dilation=d)
        assert orc.out_size(h, k, st, p, d) == t.shape[-1], (h, k, st, p, d)


# --------------------------------------------------------------------------- library routines

def _grid_sample_core(x, off, m, groups, kernel, stride, pad, dilation, s, softmax, rc=False):
    """sum_k m_k * grid_sample(x_g, location_k) in torch (fp64, autograd-able).

    x (N,H,W,C), off (N,Ho,Wo,G,K,2), m (N,Ho,Wo,G,K) are torch tensors.
    """
    n, h, w, c = x.shape
    cg = c // groups
    _, ho, wo, _, K, _ = off.shape
    mk = torch.softmax(m, dim=-1) if softmax else m
    dev = x.device
    hh = torch.arange(ho, dtype=x.dtype, device=dev).view(1, ho, 1)
    ww = torch.arange(wo, dtype=x.dtype, device=dev).view(1, 1, wo)
    outs = []
    for q in range(groups):
        xg = x[..., q * cg:(q + 1) * cg].permute(0, 3, 1, 2)          # (N, Cg, H, W)
        acc = 0.0
        for k, (i, j) in enumerate(_points(kernel, rc)):
            py = hh * stride[0] - pad[0] + i * dilation[0] + s * off[:, :, :, q, k, 1]
            px = ww * stride[1] - pad[1] + j * dilation[1] + s * off[:, :, :, q, k, 0]
            grid = torch.stack([(2 * px + 1) / w - 1, (2 * py + 1) / h - 1], dim=-1)
            samp = F.grid_sample(xg, grid, mode="bilinear", padding_mode="zeros",
                                 align_corners=False)                     # (N, Cg, Ho, Wo)
            acc = acc + mk[:, :, :, q, k].unsqueeze(1) * samp
        outs.append(acc.permute(0, 2, 3, 1))
    return torch.cat(outs, dim=-1)


_LIB_CASES = [
    dict(n=2, h=7, w=6, c=8, g=2, kernel=(3, 3), stride=(1, 1), pad=(1, 1), dilation=(1, 1), s=2.0),
    dict(n=1, h=9, w=11, c=6, g=3, kernel=(3, 3), stride=(2, 2), pad=(0, 0), dilation=(1, 1), s=2.0),
    dict(n=1, h=8, w=8, c=4, g=1, kernel=(3, 3), stride=(1, 1), pad=(2, 2), dilation=(2, 2), s=1.0),
    dict(n=1, h=6, w=9, c=10, g=2, kernel=(3, 5), stride=(1, 2), pad=(1, 2), dilation=(1, 1), s=0.5),
    # the centre point removed (DCNv4's remove_center, pnsm.cn/news/2029644.html section 3.3)
    dict(n=2, h=7, w=6, c=8, g=2, kernel=(3, 3), stride=(1, 1), pad=(1, 1), dilation=(1, 1), s=2.0,
         rc=True),
    dict(n=1, h=9, w=8, c=6, g=3, kernel=(3, 5), stride=(2, 1), pad=(1, 2), dilation=(1, 2), s=1.0,
         rc=True),
]


def pin_grid_sample_forward(orc):
    """Forward equals the grid_sample composition, for several geometries."""
    rng = np.random.default_rng(108)
    for cs in _LIB_CASES:
        for softmax in (True, False):
            rc = cs.get("rc", False)
            x, off, m = _random_case(rng, cs["n"], cs["h"], cs["w"], cs["c"], cs["g"], cs["kernel"],
                                     cs["stride"], cs["pad"], cs["dilation"], off_std=2.0, rc=rc)
            y = orc.forward(x, off, m, **_kw(cs["g"], cs["kernel"], cs["stride"], cs["pad"],
                                             cs["dilation"], cs["s"], softmax, rc))
            ref = _grid_sample_core(torch.from_numpy(x), torch.from_numpy(off), torch.from_numpy(m),
                                    cs["g"], cs["kernel"], cs["stride"], cs["pad"], cs["dilation"],
                                    cs["s"], softmax, rc)
            _close(y, ref.numpy(), 1e-12, f"grid_sample forward {cs} softmax={softmax}")


def pin_grid_sample_backward(orc):
    """Backward equals torch autograd through the grid_sample composition."""
    rng = np.random.default_rng(109)
    for cs in _LIB_CASES:
        for softmax in (True, False):
            rc = cs.get("rc", False)
            x, off, m = _random_case(rng, cs["n"], cs["h"], cs["w"], cs["c"], cs["g"], cs["kernel"],
                                     cs["stride"], cs["pad"], cs["dilation"], off_std=2.0, rc=rc)
            kw = _kw(cs["g"], cs["kernel"], cs["stride"], cs["pad"], cs["dilation"], cs["s"], softmax, rc)
            ho, wo = off.shape[1], off.shape[2]
            gy = rng.standard_normal((cs["n"], ho, wo, cs["c"]))
            gx, goff, gm = orc.backward(x, off, m, gy, **kw)
            xt, ot, mt = (torch.from_numpy(a).requires_grad_() for a in (x, off, m))
            out = _grid_sample_core(xt, ot, mt, cs["g"], cs["kernel"], cs["stride"], cs["pad"],
                                    cs["dilation"], cs["s"], softmax, rc)
            rx, ro, rm = torch.autograd.grad(out, (xt, ot, mt), grad_outputs=torch.from_numpy(gy))
            _close(gx, rx.numpy(), 1e-11, f"grad_input {cs} softmax={softmax}")
            _close(goff, ro.numpy(), 1e-10, f"grad_offset {cs} softmax={softmax}")
            _close(gm, rm.numpy(), 1e-11, f"grad_mask {cs} softmax={softmax}")


def pin_depthwise_conv(orc):
    """DCNv4 with zero offsets and a mask constant over space is a depthwise
    convolution whose tap (i, j) of channel c is mask[g(c), i*KW + j]: this
    fixes the point order (row-major, i along H), stride, pad and dilation."""
    rng = np.random.default_rng(110)
    for (n, h, w, c, g, kernel, stride, pad, dil) in [
            (2, 8, 7, 8, 2, (3, 3), (1, 1), (1, 1), (1, 1)),
            (1, 11, 9, 6, 3, (3, 3), (2, 2), (1, 0), (2, 1)),
            (1, 9, 12, 4, 1, (3, 5), (1, 2), (2, 1), (1, 2)),
            (1, 7, 7, 4, 4, (5, 3), (3, 1), (0, 2), (1, 1))]:
        ho = _out(h, kernel[0], stride[0], pad[0], dil[0])
        wo = _out(w, kernel[1], stride[1], pad[1], dil[1])
        K = kernel[0] * kernel[1]
        x = rng.standard_normal((n, h, w, c))
        mg = rng.standard_normal((g, K))
        m = np.broadcast_to(mg, (n, ho, wo, g, K)).copy()
        off = np.zeros((n, ho, wo, g, K, 2))
        y = orc.forward(x, off, m, **_kw(g, kernel, stride, pad, dil, 2.0, False))
        cg = c // g
        wt = torch.from_numpy(np.repeat(mg, cg, axis=0).reshape(c, 1, kernel[0], kernel[1]))
        ref = F.conv2d(torch.from_numpy(x).permute(0, 3, 1, 2), wt, stride=stride, padding=pad,
                       dilation=dil, groups=c).permute(0, 2, 3, 1).numpy()
        _close(y, ref, 1e-13, f"depthwise conv {kernel} {stride} {pad} {dil}")


def pin_depthwise_conv_remove_center(orc):
    """With the centre point removed, DCNv4 at zero offsets and a spatially
    constant mask is the depthwise convolution whose centre tap is zero and
    whose other taps take the K = KH*KW - 1 mask values in row-major order."""
    rng = np.random.default_rng(114)
    for (n, h, w, c, g, kernel, stride, pad, dil) in [
            (2, 8, 7, 8, 2, (3, 3), (1, 1), (1, 1), (1, 1)),
            (1, 11, 9, 6, 3, (5, 3), (2, 1), (2, 1), (1, 2)),
            (1, 9, 12, 4, 1, (3, 5), (1, 2), (1, 2), (2, 1))]:
        ho = _out(h, kernel[0], stride[0], pad[0], dil[0])
        wo = _out(w, kernel[1], stride[1], pad[1], dil[1])
        pts = _points(kernel, rc=True)
        x = rng.standard_normal((n, h, w, c))
        mg = rng.standard_normal((g, len(pts)))
        m = np.broadcast_to(mg, (n, ho, wo, g, len(pts))).copy()
        off = np.zeros((n, ho, wo, g, len(pts), 2))
        y = orc.forward(x, off, m, **_kw(g, kernel, stride, pad, dil, 2.0, False, rc=True))
        taps = np.zeros((g, kernel[0], kernel[1]))
        for k, (i, j) in enumerate(pts):
            taps[:, i, j] = mg[:, k]
        cg = c // g
        wt = torch.from_numpy(np.repeat(taps, cg, axis=0).reshape(c, 1, kernel[0], kernel[1]))
        ref = F.conv2d(torch.from_numpy(x).permute(0, 3, 1, 2), wt, stride=stride, padding=pad,
                       dilation=dil, groups=c).permute(0, 2, 3, 1).numpy()
        _close(y, ref, 1e-13, f"depthwise conv without centre {kernel} {stride} {pad} {dil}")


def _brute_forward(x, off, m, groups, kernel, stride, pad, dilation, s, softmax, rc):
    """One output element at a time, in plain Python floats, straight from the
    definition: for each point, its location on the regular grid moved by s
    times its (x, y) offset, the four floor/floor+1 neighbours weighted by
    (1 - |dy|)(1 - |dx|), zero off the map, weighted by the point's mask."""
    import math
    n_, h, w, c = x.shape
    cg = c // groups
    _, ho, wo, _, K, _ = off.shape
    pts = _points(kernel, rc)
    assert len(pts) == K
    y = np.zeros((n_, ho, wo, c))
    for n in range(n_):
        for oy in range(ho):
            for ox in range(wo):
                for g in range(groups):
                    logits = [float(m[n, oy, ox, g, k]) for k in range(K)]
                    if softmax:
                        top = max(logits)
                        e = [math.exp(v - top) for v in logits]
                        wts = [v / sum(e) for v in e]
                    else:
                        wts = logits
                    for cc in range(cg):
                        ch = g * cg + cc
                        total = 0.0
                        for k, (i, j) in enumerate(pts):
                            py = oy * stride[0] - pad[0] + i * dilation[0] + s * float(off[n, oy, ox, g, k, 1])
                            px = ox * stride[1] - pad[1] + j * dilation[1] + s * float(off[n, oy, ox, g, k, 0])
                            val = 0.0
                            for yy in (math.floor(py), math.floor(py) + 1):
                                for xx in (math.floor(px), math.floor(px) + 1):
                                    if 0 <= yy < h and 0 <= xx < w:
                                        val += (1 - abs(py - yy)) * (1 - abs(px - xx)) * float(x[n, yy, xx, ch])
                            total += wts[k] * val
                        y[n, oy, ox, ch] = total
    return y


def pin_brute_force_tiny(orc):
    """Tiny shapes against the scalar loop above: forward everywhere, and
    grad_input column by column (the forward is linear in x, so the column
    of input element e is the forward of the unit tensor at e)."""
    rng = np.random.default_rng(115)
    cases = [
        dict(h=4, w=5, c=2, g=1, kernel=(3, 3), stride=(1, 1), pad=(1, 1), dilation=(1, 1), s=2.0),
        dict(h=5, w=4, c=4, g=2, kernel=(3, 3), stride=(2, 1), pad=(0, 1), dilation=(1, 2), s=1.0),
        dict(h=4, w=4, c=2, g=2, kernel=(3, 5), stride=(1, 1), pad=(1, 2), dilation=(1, 1), s=0.5),
        dict(h=4, w=5, c=2, g=1, kernel=(3, 3), stride=(1, 1), pad=(1, 1), dilation=(1, 1), s=2.0, rc=True),
        dict(h=5, w=5, c=2, g=1, kernel=(5, 3), stride=(1, 2), pad=(2, 1), dilation=(1, 1), s=1.0, rc=True),
    ]
    for cs in cases:
        rc = cs.get("rc", False)
        for softmax in (True, False):
            x, off, m = _random_case(rng, 1, cs["h"], cs["w"], cs["c"], cs["g"], cs["kernel"], cs["stride"],
                                     cs["pad"], cs["dilation"], off_std=1.5, rc=rc)
            args = (cs["g"], cs["kernel"], cs["stride"], cs["pad"], cs["dilation"], cs["s"], softmax, rc)
            kw = _kw(*args)
            _close(orc.forward(x, off, m, **kw), _brute_forward(x, off, m, *args), 1e-13,
                   f"brute force forward {cs} softmax={softmax}")
            gy = rng.standard_normal((1, off.shape[1], off.shape[2], cs["c"]))
            gx, _, _ = orc.backward(x, off, m, gy, **kw)
            col = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                unit = np.zeros_like(x)
                unit[idx] = 1.0
                col[idx] = float(np.sum(_brute_forward(unit, off, m, *args) * gy))
            _close(gx, col, 1e-13, f"brute force grad_input {cs} softmax={softmax}")


# --------------------------------------------------------------------------- backward

def pin_adjoint(orc):
    """grad_input is the adjoint of the (linear in x) forward:
    <F(x), g> = <x, F^T(g)>, for both mask kinds."""
    rng = np.random.default_rng(111)
    for softmax in (True, False):
        x, off, m = _random_case(rng, 2, 8, 7, 12, 3, off_std=2.0)
        gy = rng.standard_normal((2, 8, 7, 12))
        kw = _kw(3, softmax=softmax)
        lhs = float(np.sum(orc.forward(x, off, m, **kw) * gy))
        gx, _, _ = orc.backward(x, off, m, gy, **kw)
        rhs = float(np.sum(x * gx))
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)), (lhs, rhs)


def pin_finite_differences(orc):
    """grad_offset and grad_mask match central differences of the forward
    (fp64, h = 1e-6, every sample kept at least 0.1 px from a kink)."""
    rng = np.random.default_rng(112)
    n, h, w, c, g, s = 1, 5, 6, 6, 2, 2.0
    for softmax in (True, False):
        K = 9
        # s*offset = integer + fraction in [0.1, 0.9]: no floor boundary within reach
        whole = rng.integers(-3, 4, size=(n, h, w, g, K, 2))
        frac = rng.uniform(0.1, 0.9, size=(n, h, w, g, K, 2))
        off = (whole + frac) / s
        x = rng.standard_normal((n, h, w, c))
        m = rng.standard_normal((n, h, w, g, K))
        gy = rng.standard_normal((n, h, w, c))
        kw = _kw(g, s=s, softmax=softmax)
        _, goff, gm = orc.backward(x, off, m, gy, **kw)

        def loss(o, mm):
            return float(np.sum(orc.forward(x, o, mm, **kw) * gy))

        step = 1e-6
        fd = np.zeros_like(off)
        for idx in np.ndindex(off.shape):
            o1 = off.copy()
            o2 = off.copy()
            o1[idx] += step
            o2[idx] -= step
            fd[idx] = (loss(o1, m) - loss(o2, m)) / (2 * step)
        _close(goff, fd, 1e-7, f"grad_offset vs finite differences (softmax={softmax})")
        fdm = np.zeros_like(m)
        for idx in np.ndindex(m.shape):
            m1 = m.copy()
            m2 = m.copy()
            m1[idx] += step
            m2[idx] -= step
            fdm[idx] = (loss(off, m1) - loss(off, m2)) / (2 * step)
        _close(gm, fdm, 1e-7, f"grad_mask vs finite differences (softmax={softmax})")


def pin_softmax_grad_sums_to_zero(orc):
    """Through a softmax the logit gradients of one (pixel, group) sum to 0."""
    rng = np.random.default_rng(113)
    x, off, m = _random_case(rng, 2, 6, 6, 8, 2)
    gy = rng.standard_normal((2, 6, 6, 8))
    _, _, gm = orc.backward(x, off, m, gy, **_kw(2, softmax=True))
    assert np.max(np.abs(gm.sum(axis=-1))) < 1e-13
    assert np.max(np.abs(gm)) > 1e-3


def pin_backward_far_away_is_zero(orc):
    """Zero padding in the backward (wmrh.cn/news/61976 section 二 step 4: the
    sample reads zeros off the map).  A sample off the map has B = 0 and
    dB = 0, so it scatters nothing into grad_input, its offset gradient
    s * m_k * 0 is 0, its gm_k is 0, and through the DCNv3 softmax Jacobian
    m_k * (0 - sum_j m_j * 0) = 0 as well.  Offsets of +-1e4 (far, through the
    ordinary corner path), +-1e300 and +-Inf (beyond any representable map),
    on both axes or only one of them."""
    rng = np.random.default_rng(114)
    n, h, w, c, g = 1, 6, 5, 8, 2
    x = rng.standard_normal((n, h, w, c))
    m = rng.standard_normal((n, h, w, g, 9))
    gy = rng.standard_normal((n, h, w, c))
    for big in (1e4, -1e4, 1e300, -1e300, np.inf, -np.inf):
        for axes in ((0, 1), (0,), (1,)):
            off = rng.standard_normal((n, h, w, g, 9, 2))
            for a in axes:
                off[..., a] = big
            for softmax in (True, False):
                kw = _kw(g, softmax=softmax)
                what = f"offset {big} on axes {axes}, softmax={softmax}"
                y = orc.forward(x, off, m, **kw)
                assert np.all(y == 0.0), f"forward, {what}: not exactly zero"
                gx, goff, gm = orc.backward(x, off, m, gy, **kw)
                assert np.all(gx == 0.0), f"grad_input, {what}: not exactly zero"
                assert np.all(goff == 0.0), f"grad_offset, {what}: not exactly zero"
                assert np.all(gm == 0.0), f"grad_mask, {what}: not exactly zero"
    # one far point in an otherwise ordinary problem: its rows are zero and the
    # rest equals the problem with that point's weight set to zero (DCNv4: the
    # raw mask; DCNv3: the softmax weights computed here by scipy and passed
    # as raw weights, the far point's zeroed)
    x, off, m = _random_case(rng, 1, 6, 5, 8, 2, off_std=1.5)
    gy = rng.standard_normal((1, 6, 5, 8))
    at = (0, 2, 3, 1, 5)
    off[at + (1,)] = np.inf
    for softmax in (True, False):
        gx, goff, gm = orc.backward(x, off, m, gy, **_kw(2, softmax=softmax))
        assert np.all(goff[at] == 0.0), f"far point's grad_offset (softmax={softmax})"
        wts = scipy.special.softmax(m, axis=-1) if softmax else m.copy()
        wts[at] = 0.0
        off0 = off.copy()
        off0[at] = 0.0
        rx, roff, rgm = orc.backward(x, off0, wts, gy, **_kw(2, softmax=False))
        _close(gx, rx, 1e-12, f"grad_input with one far point (softmax={softmax})")
        keep = np.ones(off.shape[:-1], dtype=bool)
        keep[at] = False
        _close(goff[keep], roff[keep], 1e-12, f"grad_offset of the other points (softmax={softmax})")
        if softmax:  # gm of the far point is 0; the Jacobian of the scipy softmax
            sm = scipy.special.softmax(m, axis=-1)
            raw = rgm.copy()
            raw[at] = 0.0
            ref = sm * (raw - np.sum(sm * raw, axis=-1, keepdims=True))
            _close(gm, ref, 1e-12, "grad_mask with one far point (softmax)")
        else:
            assert gm[at] == 0.0, "far point's gm (DCNv4)"
            _close(gm[keep], rgm[keep], 1e-12, "grad_mask of the other points (DCNv4)")


def pin_backward_nan_offset_is_local(orc):
    """A NaN offset makes its sampling location NaN.  Reading taken: the
    sample's gradients are NaN (its grad_offset pair and gm_k, and for DCNv3
    every logit gradient of its (pixel, group), through the softmax Jacobian's
    sum over the points) and it scatters nothing into grad_input.  Every other
    gradient is that of the same problem with the point's weight set to zero:
    checked against the oracle run on raw weights (the DCNv3 softmax computed
    here by scipy), the Jacobian applied here for DCNv3."""
    rng = np.random.default_rng(115)
    x, off, m = _random_case(rng, 1, 6, 5, 8, 2, off_std=1.5)
    gy = rng.standard_normal((1, 6, 5, 8))
    at = (0, 2, 3, 1, 4)
    off[at + (0,)] = np.nan
    for softmax in (True, False):
        gx, goff, gm = orc.backward(x, off, m, gy, **_kw(2, softmax=softmax))
        assert np.all(np.isnan(goff[at])), f"NaN point's grad_offset (softmax={softmax})"
        wts = scipy.special.softmax(m, axis=-1) if softmax else m.copy()
        wts[at] = 0.0
        off0 = off.copy()
        off0[at] = 0.0
        rx, roff, rgm = orc.backward(x, off0, wts, gy, **_kw(2, softmax=False))
        assert np.all(np.isfinite(gx)), f"NaN reached grad_input (softmax={softmax})"
        _close(gx, rx, 1e-12, f"grad_input beside a NaN point (softmax={softmax})")
        keep = np.ones(off.shape[:-1], dtype=bool)
        keep[at] = False
        _close(goff[keep], roff[keep], 1e-12, f"grad_offset beside a NaN point (softmax={softmax})")
        if softmax:
            assert np.all(np.isnan(gm[at[:4]])), "the NaN point's group: every logit gradient NaN"
            other = np.ones(m.shape[:-1], dtype=bool)
            other[at[:4]] = False
            sm = scipy.special.softmax(m, axis=-1)
            ref = sm * (rgm - np.sum(sm * rgm, axis=-1, keepdims=True))
            _close(gm[other], ref[other], 1e-12, "grad_mask of the other (pixel, group)s (softmax)")
        else:
            assert np.isnan(gm[at]), "the NaN point's gm (DCNv4)"
            assert np.sum(np.isnan(gm)) == 1, "NaN leaked into other mask gradients (DCNv4)"
            _close(gm[keep], rgm[keep], 1e-12, "grad_mask beside a NaN point (DCNv4)")


# --------------------------------------------------------------------------- the steps before and after

def pin_linear_is_matmul(orc):
    """The oracle's linear layer equals a library matrix product, x w^T + b,
    over any leading shape, with and without a bias."""
    rng = np.random.default_rng(120)
    for shape, nin, nout in [((5,), 7, 3), ((2, 3, 4), 16, 54), ((1,), 1, 1)]:
        x = rng.standard_normal(shape + (nin,))
        w = rng.standard_normal((nout, nin))
        b = rng.standard_normal(nout)
        _close(orc.linear(x, w, b), np.matmul(x, w.T) + b, 1e-12, f"linear {shape} {nin}->{nout}")
        _close(orc.linear(x, w, None), np.matmul(x, w.T), 1e-12, f"linear without bias {shape}")


def _om_case(rng, n, h, w, c, g, cgd, kernel=(3, 3), stride=(1, 1), pad=(1, 1), dilation=(1, 1), rc=False,
             wscale=0.3):
    ho = _out(h, kernel[0], stride[0], pad[0], dilation[0])
    wo = _out(w, kernel[1], stride[1], pad[1], dilation[1])
    K = len(_points(kernel, rc))
    x = rng.standard_normal((n, h, w, c))
    guide = rng.standard_normal((n, ho, wo, cgd))
    w_off = rng.standard_normal((g * K * 2, cgd)) * wscale
    b_off = rng.standard_normal(g * K * 2)
    w_mask = rng.standard_normal((g * K, cgd)) * wscale
    b_mask = rng.standard_normal(g * K)
    return x, guide, w_off, b_off, w_mask, b_mask


def pin_generation_zero_weights_is_box_average(orc):
    """With the generation weights and biases all zero (the initialisation
    the pages describe, wmrh.cn/news/61976 section 二, the "细节亮点" note:
    offsets and mask start at zero, so the operator starts as a plain 3x3
    convolution) the offsets are 0 and the logits 0: DCNv3 is then the
    zero-padded 3x3 box average of x, whatever the guide."""
    rng = np.random.default_rng(121)
    n, h, w, c, g, cgd = 2, 7, 6, 32, 2, 24
    x, guide, w_off, b_off, w_mask, b_mask = _om_case(rng, n, h, w, c, g, cgd)
    z = lambda a: np.zeros_like(a)
    y = orc.forward_om(x, guide, z(w_off), z(b_off), z(w_mask), z(b_mask), **_kw(g))
    xt = torch.from_numpy(x).permute(0, 3, 1, 2)
    ref = F.avg_pool2d(xt, 3, stride=1, padding=1, count_include_pad=True).permute(0, 2, 3, 1).numpy()
    _close(y, ref, 1e-14, "generation with zero weights")
    y0 = orc.forward_om(x, guide, z(w_off), None, z(w_mask), None, **_kw(g))
    _close(y0, ref, 1e-14, "generation with zero weights and no biases")


def pin_generation_is_linear_then_core(orc):
    """forward_om equals torch's F.linear for the two branches, reshaped to
    (N, Ho, Wo, G, K, 2) and (N, Ho, Wo, G, K), fed to the grid_sample
    composition of the core (fp64 torch), over several geometries, both mask
    kinds and without the centre."""
    rng = np.random.default_rng(122)
    for cs in _LIB_CASES:
        rc = cs.get("rc", False)
        for softmax in (True, False):
            cgd = 12
            x, guide, w_off, b_off, w_mask, b_mask = _om_case(
                rng, cs["n"], cs["h"], cs["w"], cs["c"], cs["g"], cgd, cs["kernel"], cs["stride"], cs["pad"],
                cs["dilation"], rc)
            kw = _kw(cs["g"], cs["kernel"], cs["stride"], cs["pad"], cs["dilation"], cs["s"], softmax, rc)
            y = orc.forward_om(x, guide, w_off, b_off, w_mask, b_mask, **kw)
            gt = torch.from_numpy(guide)
            n, ho, wo, _ = guide.shape
            K = len(_points(cs["kernel"], rc))
            off = F.linear(gt, torch.from_numpy(w_off), torch.from_numpy(b_off)).reshape(n, ho, wo, cs["g"], K, 2)
            m = F.linear(gt, torch.from_numpy(w_mask), torch.from_numpy(b_mask)).reshape(n, ho, wo, cs["g"], K)
            ref = _grid_sample_core(torch.from_numpy(x), off, m, cs["g"], cs["kernel"], cs["stride"], cs["pad"],
                                    cs["dilation"], cs["s"], softmax, rc)
            _close(y, ref.numpy(), 1e-12, f"generation then core {cs} softmax={softmax}")


def pin_generation_brute_force_tiny(orc):
    """Tiny shapes: each offset component and mask value summed term by term
    in plain Python floats from the weights' (out, in) layout, then the
    scalar forward loop."""
    rng = np.random.default_rng(123)
    for cs in [dict(h=4, w=5, c=2, g=1, cgd=3, kernel=(3, 3), rc=False),
               dict(h=3, w=4, c=4, g=2, cgd=5, kernel=(3, 3), rc=True)]:
        for softmax in (True, False):
            x, guide, w_off, b_off, w_mask, b_mask = _om_case(rng, 1, cs["h"], cs["w"], cs["c"], cs["g"], cs["cgd"],
                                                               cs["kernel"], rc=cs["rc"])
            n, ho, wo, cgd = guide.shape
            K = len(_points(cs["kernel"], cs["rc"]))
            off = np.zeros((n, ho, wo, cs["g"], K, 2))
            m = np.zeros((n, ho, wo, cs["g"], K))
            for oy in range(ho):
                for ox in range(wo):
                    for g in range(cs["g"]):
                        for k in range(K):
                            for e in range(2):
                                row = (g * K + k) * 2 + e
                                off[0, oy, ox, g, k, e] = float(b_off[row]) + sum(
                                    float(guide[0, oy, ox, q]) * float(w_off[row, q]) for q in range(cgd))
                            row = g * K + k
                            m[0, oy, ox, g, k] = float(b_mask[row]) + sum(
                                float(guide[0, oy, ox, q]) * float(w_mask[row, q]) for q in range(cgd))
            args = (cs["g"], cs["kernel"], (1, 1), (1, 1), (1, 1), 2.0, softmax, cs["rc"])
            ref = _brute_forward(x, off, m, *args)
            _close(orc.forward_om(x, guide, w_off, b_off, w_mask, b_mask, **_kw(*args)), ref, 1e-12,
                   f"generation brute force {cs} softmax={softmax}")


def pin_output_projection(orc):
    """forward_proj equals torch's F.linear applied to the grid_sample
    composition of the core; the identity projection returns the core's
    output, a channel permutation permutes it."""
    rng = np.random.default_rng(124)
    for cs in _LIB_CASES[:3] + _LIB_CASES[4:5]:
        rc = cs.get("rc", False)
        for softmax in (True, False):
            x, off, m = _random_case(rng, cs["n"], cs["h"], cs["w"], cs["c"], cs["g"], cs["kernel"], cs["stride"],
                                     cs["pad"], cs["dilation"], off_std=2.0, rc=rc)
            c = cs["c"]
            w_out = rng.standard_normal((c, c))
            b_out = rng.standard_normal(c)
            kw = _kw(cs["g"], cs["kernel"], cs["stride"], cs["pad"], cs["dilation"], cs["s"], softmax, rc)
            core = _grid_sample_core(torch.from_numpy(x), torch.from_numpy(off), torch.from_numpy(m), cs["g"],
                                     cs["kernel"], cs["stride"], cs["pad"], cs["dilation"], cs["s"], softmax, rc)
            ref = F.linear(core, torch.from_numpy(w_out), torch.from_numpy(b_out)).numpy()
            _close(orc.forward_proj(x, off, m, w_out, b_out, **kw), ref, 1e-12, f"projection {cs} softmax={softmax}")
            _close(orc.forward_proj(x, off, m, np.eye(c), None, **kw), core.numpy(), 1e-13, "identity projection")
            perm = rng.permutation(c)
            _close(orc.forward_proj(x, off, m, np.eye(c)[perm], None, **kw), core.numpy()[..., perm], 1e-13,
                   "permutation projection")


ALL_PINS = [
    pin_box_average, pin_integer_offsets_exact_gather, pin_partition_of_unity,
    pin_out_of_range_is_zero, pin_backward_far_away_is_zero, pin_backward_nan_offset_is_local,
    pin_hand_golden, pin_linearity, pin_group_independence,
    pin_forward_pixels, pin_out_size, pin_grid_sample_forward, pin_grid_sample_backward,
    pin_depthwise_conv, pin_depthwise_conv_remove_center, pin_brute_force_tiny, pin_adjoint, pin_finite_differences, pin_softmax_grad_sums_to_zero,
    pin_linear_is_matmul, pin_generation_zero_weights_is_box_average, pin_generation_is_linear_then_core,
    pin_generation_brute_force_tiny, pin_output_projection,
]
