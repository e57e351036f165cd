"""Pins for the CPU oracle, each against something other than the oracle itself.

  * dense index-grid brute force for the neighbour map (tiny grids);
  * the closed form (3L - 2d)^3 for the valid pairs of a full L^3 cube;
  * map invariants: centre offset is the identity, offsets k and K-1-k mirror;
  * torch.nn.functional.conv3d in float64 on the dense grid, sampled at the
    active sites (fixes the offset numbering and direction against a library
    routine);
  * K=1 reduces to a plain GEMM (numpy float64 matmul);
  * an all-sentinel map returns the bias;
  * feats = w = 1 gives bias + Ci * (number of present neighbours);
  * linearity in feats and in w (exact with small-integer data);
  * bf16 inputs are widened exactly;
  * a hand-worked three-voxel example (tests/golden);
  * Morton codes against a bit-by-bit interleave and closed forms;
  * the input gradient against torch autograd through float64 conv3d on the
    dense grid, the adjoint identity <forward(x), y> = <x, dgrad(y)>, the K=1
    GEMM transpose, and the mirrored-map form the GPU uses;
  * the weight gradient against torch autograd through float64 conv3d, the
    identity <dw, W> = <forward_W(feats), dout>, and the K=1 product feats^T dout;
  * the float32 -> bfloat16 cast against hand-worked ties, overflow, subnormal
    and NaN cases and against torch's own conversion on every class of bit
    pattern; bfloat16 -> float32 on all 65536 patterns; the mixed-dtype forward
    through K=1 identity weights (output = the cast features) and against the
    same-dtype forward where the cast is exact.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def offsets(K, dilation):
    s = round(K ** (1.0 / 3.0))
    r = (s - 1) // 2
    out = []
    for a in range(s):
        for b in range(s):
            for c in range(s):
                out.append(((a - r) * dilation, (b - r) * dilation, (c - r) * dilation))
    return np.array(out, dtype=np.int64)


def random_sites(rng, G, density, origin=(0, 0, 0)):
    m = rng.random((G, G, G)) < density
    c = np.argwhere(m).astype(np.int64) + np.array(origin, dtype=np.int64)
    perm = rng.permutation(c.shape[0])
    return c[perm].astype(np.int32)


def brute_nmap(coords, K, dilation):
    """Dense index grid lookup: idx[x,y,z] = voxel number or -1."""
    c = coords.astype(np.int64)
    N = c.shape[0]
    lo = c.min(0) - 8 * dilation
    hi = c.max(0) + 8 * dilation
    shape = tuple((hi - lo + 1).tolist())
    idx = -np.ones(shape, dtype=np.int64)
    idx[tuple((c - lo).T)] = np.arange(N)
    out = np.full((K, N), N, dtype=np.int32)
    for k, o in enumerate(offsets(K, dilation)):
        q = c + o - lo
        m = idx[tuple(q.T)]
        out[k] = np.where(m >= 0, m, N)
    return out


@pytest.mark.parametrize("G,density,K,d", [(6, 0.5, 27, 1), (10, 0.2, 27, 2), (9, 0.35, 125, 1),
                                           (12, 0.1, 27, 3), (7, 0.6, 1, 1), (16, 0.05, 125, 2)])
def test_nmap_matches_dense_grid_bruteforce(G, density, K, d):
    rng = np.random.default_rng(G * 1000 + K + d)
    coords = random_sites(rng, G, density, origin=(-3, 5, -7))
    assert np.array_equal(oracle.nmap(coords, K, d), brute_nmap(coords, K, d))


def test_nmap_rows_is_column_subset():
    rng = np.random.default_rng(7)
    coords = random_sites(rng, 12, 0.3)
    full = oracle.nmap(coords, 27, 1)
    rows = rng.choice(coords.shape[0], 50, replace=False)
    assert np.array_equal(oracle.nmap_rows(coords, rows, 27, 1), full[:, rows])


def test_coordinate_range_edges():
    # neighbours falling outside [-2^20, 2^20) are simply missing
    B = 1 << 20
    coords = np.array([[-B, 0, 0], [-B + 1, 0, 0], [B - 1, 5, 5], [B - 2, 5, 5]], dtype=np.int32)
    nb = oracle.nmap(coords, 27, 1)
    assert nb[13].tolist() == [0, 1, 2, 3]
    assert nb[22, 0] == 1 and nb[4, 1] == 0          # (+1,0,0) and (-1,0,0)
    assert nb[4, 2] == 3 and nb[22, 3] == 2
    assert nb[4, 0] == 4 and nb[22, 2] == 4          # beyond the range: sentinel
    assert brute_nmap(coords, 27, 1).tolist() == nb.tolist()


@pytest.mark.parametrize("L,d", [(8, 1), (8, 2), (11, 1), (11, 3)])
def test_full_cube_valid_pairs_closed_form(L, d):
    g = np.arange(L)
    coords = np.stack(np.meshgrid(g, g, g, indexing="ij"), -1).reshape(-1, 3).astype(np.int32)
    nb = oracle.nmap(coords, 27, d)
    N = coords.shape[0]
    assert int((nb != N).sum()) == (3 * L - 2 * d) ** 3


def test_nmap_invariants():
    rng = np.random.default_rng(3)
    for K, d in [(27, 1), (27, 2), (125, 1)]:
        coords = random_sites(rng, 14, 0.25)
        N = coords.shape[0]
        nb = oracle.nmap(coords, K, d)
        assert np.array_equal(nb[(K - 1) // 2], np.arange(N))
        for k in range(K):
            v = nb[k]
            ok = v != N
            # nbr[k,n] = m  <=>  nbr[K-1-k, m] = n
            assert np.array_equal(nb[K - 1 - k][v[ok]], np.arange(N)[ok])
        assert ((nb >= 0) & (nb <= N)).all()


def test_nmap_errors():
    dup = np.array([[0, 0, 0], [1, 1, 1], [0, 0, 0]], dtype=np.int32)
    with pytest.raises(oracle.OracleError) as e:
        oracle.nmap(dup, 27, 1)
    assert e.value.code == -4
    far = np.array([[0, 0, 1 << 20]], dtype=np.int32)
    with pytest.raises(oracle.OracleError) as e:
        oracle.nmap(far, 27, 1)
    assert e.value.code == -3
    for K in (0, 8, 26, 64):
        with pytest.raises(oracle.OracleError):
            oracle.nmap(dup[:2], K, 1)
    with pytest.raises(oracle.OracleError):
        oracle.nmap(dup[:2], 27, 0)


def dense_conv_reference(coords, feats, w, bias, K, d):
    """conv3d (cross-correlation) in float64 on the dense grid, read at the sites."""
    s = round(K ** (1.0 / 3.0))
    r = (s - 1) // 2
    c = coords.astype(np.int64)
    lo = c.min(0)
    G = tuple((c.max(0) - lo + 1).tolist())
    Ci = feats.shape[1]
    Co = w.shape[2]
    grid = torch.zeros((1, Ci) + G, dtype=torch.float64)
    q = c - lo
    grid[0, :, q[:, 0], q[:, 1], q[:, 2]] = torch.from_numpy(feats.astype(np.float64)).T
    # weight[co, ci, a, b, c] = w[(a*s + b)*s + c, ci, co]
    wt = torch.from_numpy(w.astype(np.float64)).reshape(s, s, s, Ci, Co).permute(4, 3, 0, 1, 2).contiguous()
    y = torch.nn.functional.conv3d(grid, wt, torch.from_numpy(bias.astype(np.float64)),
                                   padding=d * r, dilation=d)
    return y[0, :, q[:, 0], q[:, 1], q[:, 2]].T.numpy()


@pytest.mark.parametrize("G,density,K,d,Ci,Co", [(8, 0.3, 27, 1, 3, 4), (10, 0.25, 27, 2, 5, 2),
                                                 (9, 0.4, 125, 1, 2, 3), (6, 0.5, 1, 1, 4, 6)])
def test_forward_matches_dense_conv3d(G, density, K, d, Ci, Co):
    rng = np.random.default_rng(11 + G + K + d)
    coords = random_sites(rng, G, density)
    N = coords.shape[0]
    feats = rng.standard_normal((N, Ci)).astype(np.float32)
    w = rng.standard_normal((K, Ci, Co)).astype(np.float32)
    bias = rng.standard_normal(Co).astype(np.float32)
    nb = oracle.nmap(coords, K, d)
    out, sab = oracle.forward(feats, nb, w, bias)
    ref = dense_conv_reference(coords, feats, w, bias, K, d)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-11 * (1 + np.abs(ref).max()))
    assert (sab >= np.abs(out - bias.astype(np.float64)) - 1e-12).all()


def test_k1_reduces_to_gemm():
    rng = np.random.default_rng(5)
    N, Ci, Co = 300, 32, 48
    coords = random_sites(rng, 20, 0.05)[:N]
    N = coords.shape[0]
    feats = rng.standard_normal((N, Ci)).astype(np.float32)
    w = rng.standard_normal((1, Ci, Co)).astype(np.float32)
    bias = rng.standard_normal(Co).astype(np.float32)
    nb = oracle.nmap(coords, 1, 1)
    assert np.array_equal(nb[0], np.arange(N))
    out = oracle.forward(feats, nb, w, bias, with_abs=False)
    ref = feats.astype(np.float64) @ w[0].astype(np.float64) + bias.astype(np.float64)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-12)


def test_all_sentinel_returns_bias():
    rng = np.random.default_rng(6)
    N, Ci, Co, K = 77, 16, 24, 27
    feats = rng.standard_normal((N, Ci)).astype(np.float32)
    w = rng.standard_normal((K, Ci, Co)).astype(np.float32)
    bias = rng.standard_normal(Co).astype(np.float32)
    for fill in (N, N + 5, -1, np.iinfo(np.int32).max):
        nb = np.full((K, N), fill, dtype=np.int32)
        out, sab = oracle.forward(feats, nb, w, bias)
        assert (out == bias.astype(np.float64)[None, :]).all()
        assert (sab == 0).all()
    out = oracle.forward(feats, np.full((K, N), N, np.int32), w, None, with_abs=False)
    assert (out == 0).all()


def test_ones_count_neighbours():
    rng = np.random.default_rng(8)
    coords = random_sites(rng, 10, 0.3)
    N = coords.shape[0]
    Ci, Co = 7, 5
    nb = oracle.nmap(coords, 27, 1)
    bias = np.arange(Co, dtype=np.float32) * 0.25
    out = oracle.forward(np.ones((N, Ci), np.float32), nb, np.ones((27, Ci, Co), np.float32), bias,
                         with_abs=False)
    v = (nb != N).sum(0).astype(np.float64)
    assert (out == bias[None, :].astype(np.float64) + Ci * v[:, None]).all()


def test_linearity_exact_with_integers():
    rng = np.random.default_rng(9)
    coords = random_sites(rng, 9, 0.4)
    N = coords.shape[0]
    Ci, Co, K = 6, 4, 27
    nb = oracle.nmap(coords, K, 1)
    f1 = rng.integers(-8, 9, (N, Ci)).astype(np.float32)
    f2 = rng.integers(-8, 9, (N, Ci)).astype(np.float32)
    w1 = rng.integers(-8, 9, (K, Ci, Co)).astype(np.float32)
    w2 = rng.integers(-8, 9, (K, Ci, Co)).astype(np.float32)
    F = lambda f, w: oracle.forward(f, nb, w, None, with_abs=False)
    assert (F(2 * f1 - 3 * f2, w1) == 2 * F(f1, w1) - 3 * F(f2, w1)).all()
    assert (F(f1, 2 * w1 - 3 * w2) == 2 * F(f1, w1) - 3 * F(f1, w2)).all()


def test_bf16_inputs_widen_exactly():
    rng = np.random.default_rng(10)
    coords = random_sites(rng, 10, 0.3)
    N = coords.shape[0]
    nb = oracle.nmap(coords, 27, 1)
    fb = torch.from_numpy(rng.standard_normal((N, 8)).astype(np.float32)).to(torch.bfloat16)
    wb = torch.from_numpy(rng.standard_normal((27, 8, 3)).astype(np.float32)).to(torch.bfloat16)
    bias = torch.randn(3, generator=torch.Generator().manual_seed(0))
    a = oracle.forward(fb, nb, wb, bias, with_abs=False)
    b = oracle.forward(fb.float(), nb, wb.float(), bias, with_abs=False)
    assert (a == b).all()


def test_handworked_golden_example():
    with open(os.path.join(GOLDEN, "handworked_three_voxels.json")) as fh:
        g = json.load(fh)
    coords = np.array(g["coords"], dtype=np.int32)
    N = coords.shape[0]
    K = g["K"]
    feats = np.array(g["feats"], dtype=np.float32)
    w = (np.arange(K, dtype=np.float32) + 1).reshape(K, 1, 1)
    bias = np.array(g["bias"], dtype=np.float32)
    for case in g["cases"]:
        nb = oracle.nmap(coords, K, case["dilation"])
        expect = np.full((K, N), N, dtype=np.int32)
        for k, n, m in case["nbr_nonsentinel"]:
            expect[k, n] = m
        assert np.array_equal(nb, expect), case["dilation"]
        out = oracle.forward(feats, nb, w, bias, with_abs=False)
        assert out[:, 0].tolist() == case["out"]
    gc = g["gemm_case"]
    out = oracle.forward(np.array(gc["feats"], np.float32), np.zeros((1, 1), np.int32),
                         np.array(gc["w0"], np.float32)[None], np.array(gc["bias"], np.float32),
                         with_abs=False)
    assert out[0].tolist() == gc["out"]


def test_morton_codes():
    B = 1 << 20
    base = np.array([-B, -B, -B], dtype=np.int64)
    pts = np.array([[1, 0, 0], [0, 1, 0], [0, 0, 1], [3, 3, 3], [0, 0, 0]], dtype=np.int64) + base
    assert oracle.morton(pts.astype(np.int32)).tolist() == [4, 2, 1, 63, 0]
    rng = np.random.default_rng(12)
    c = rng.integers(-B, B, (200, 3)).astype(np.int32)
    got = oracle.morton(c)
    for i in range(c.shape[0]):
        bx, by, bz = (int(v) + B for v in c[i])
        code = 0
        for b in range(21):
            code |= ((bz >> b) & 1) << (3 * b)
            code |= ((by >> b) & 1) << (3 * b + 1)
            code |= ((bx >> b) & 1) << (3 * b + 2)
        assert int(got[i]) == code


# ---------------------------------------------------------------------------
# input gradient (dgrad)
# ---------------------------------------------------------------------------
def dense_conv_input_grad(coords, dout, w, K, d):
    """Gradient of sum(conv3d(grid) * G) with respect to the dense input grid,
    read at the sites, where G holds dout at the sites and 0 elsewhere (a
    submanifold convolution has outputs only at the sites)."""
    s = round(K ** (1.0 / 3.0))
    r = (s - 1) // 2
    c = coords.astype(np.int64)
    lo = c.min(0)
    G = tuple((c.max(0) - lo + 1).tolist())
    Co = dout.shape[1]
    Ci = w.shape[1]
    q = c - lo
    grid = torch.zeros((1, Ci) + G, dtype=torch.float64, requires_grad=True)
    wt = torch.from_numpy(w.astype(np.float64)).reshape(s, s, s, Ci, Co).permute(4, 3, 0, 1, 2).contiguous()
    y = torch.nn.functional.conv3d(grid, wt, None, padding=d * r, dilation=d)
    g = torch.zeros_like(y)
    g[0, :, q[:, 0], q[:, 1], q[:, 2]] = torch.from_numpy(dout.astype(np.float64)).T
    (y * g).sum().backward()
    return grid.grad[0, :, q[:, 0], q[:, 1], q[:, 2]].T.numpy()


@pytest.mark.parametrize("G,density,K,d,Ci,Co", [(8, 0.3, 27, 1, 3, 4), (10, 0.25, 27, 2, 5, 2),
                                                 (9, 0.4, 125, 1, 2, 3), (6, 0.5, 1, 1, 4, 6)])
def test_dgrad_matches_conv3d_autograd(G, density, K, d, Ci, Co):
    rng = np.random.default_rng(23 + G + K + d)
    coords = random_sites(rng, G, density)
    N = coords.shape[0]
    dout = rng.standard_normal((N, Co)).astype(np.float32)
    w = rng.standard_normal((K, Ci, Co)).astype(np.float32)
    nb = oracle.nmap(coords, K, d)
    got, sab = oracle.dgrad(dout, nb, w)
    ref = dense_conv_input_grad(coords, dout, w, K, d)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11 * (1 + np.abs(ref).max()))
    assert (sab >= np.abs(got) - 1e-12).all()


def test_dgrad_adjoint_identity():
    rng = np.random.default_rng(29)
    coords = random_sites(rng, 14, 0.2)
    N, K, Ci, Co = coords.shape[0], 27, 6, 5
    x = rng.standard_normal((N, Ci)).astype(np.float32)
    y = rng.standard_normal((N, Co)).astype(np.float32)
    w = rng.standard_normal((K, Ci, Co)).astype(np.float32)
    nb = oracle.nmap(coords, K, 1)
    lhs = float((oracle.forward(x, nb, w, None, with_abs=False) * y.astype(np.float64)).sum())
    rhs = float((x.astype(np.float64) * oracle.dgrad(y, nb, w, with_abs=False)).sum())
    assert abs(lhs - rhs) <= 1e-11 * (abs(lhs) + 1.0)


def test_dgrad_k1_is_transposed_gemm_and_rows_subset():
    rng = np.random.default_rng(31)
    coords = random_sites(rng, 20, 0.04)
    N, Ci, Co = coords.shape[0], 16, 24
    dout = rng.standard_normal((N, Co)).astype(np.float32)
    w = rng.standard_normal((1, Ci, Co)).astype(np.float32)
    nb = oracle.nmap(coords, 1, 1)
    got = oracle.dgrad(dout, nb, w, with_abs=False)
    np.testing.assert_allclose(got, dout.astype(np.float64) @ w[0].astype(np.float64).T, rtol=1e-13, atol=1e-12)
    rows = rng.choice(N, 17, replace=False)
    sub = oracle.dgrad(dout, nb, w, rows=rows, with_abs=False)
    assert np.array_equal(sub, got[rows])


def test_dgrad_equals_forward_on_mirrored_weights():
    # A map built from a symmetric stencil is its own mirror: nbr[K-1-k, nbr[k, n]] = n.
    # dgrad is then the forward with w'[k] = w[K-1-k]^T (the form the GPU path runs).
    rng = np.random.default_rng(37)
    coords = random_sites(rng, 12, 0.3)
    N, K, Ci, Co = coords.shape[0], 27, 4, 7
    dout = rng.standard_normal((N, Co)).astype(np.float32)
    w = rng.standard_normal((K, Ci, Co)).astype(np.float32)
    for d in (1, 2):
        nb = oracle.nmap(coords, K, d)
        wm = np.ascontiguousarray(w[::-1].transpose(0, 2, 1))
        a = oracle.dgrad(dout, nb, w, with_abs=False)
        b = oracle.forward(dout, nb, wm, None, with_abs=False)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * (1 + np.abs(a).max()))


# ---------------------------------------------------------------------------
# weight gradient (wgrad)
# ---------------------------------------------------------------------------
def dense_conv_weight_grad(coords, feats, dout, K, d, Co):
    """Gradient of sum(conv3d(grid, W) * G) with respect to W, as (K, Ci, Co),
    where grid holds feats at the sites and G holds dout at the sites."""
    s = round(K ** (1.0 / 3.0))
    r = (s - 1) // 2
    c = coords.astype(np.int64)
    lo = c.min(0)
    G = tuple((c.max(0) - lo + 1).tolist())
    Ci = feats.shape[1]
    q = c - lo
    grid = torch.zeros((1, Ci) + G, dtype=torch.float64)
    grid[0, :, q[:, 0], q[:, 1], q[:, 2]] = torch.from_numpy(feats.astype(np.float64)).T
    wt = torch.zeros((Co, Ci, s, s, s), dtype=torch.float64, requires_grad=True)
    y = torch.nn.functional.conv3d(grid, wt, None, padding=d * r, dilation=d)
    g = torch.zeros_like(y)
    g[0, :, q[:, 0], q[:, 1], q[:, 2]] = torch.from_numpy(dout.astype(np.float64)).T
    (y * g).sum().backward()
    # weight[co, ci, a, b, c] <-> w[(a*s + b)*s + c, ci, co]
    return wt.grad.permute(2, 3, 4, 1, 0).reshape(K, Ci, Co).numpy()


@pytest.mark.parametrize("G,density,K,d,Ci,Co", [(8, 0.3, 27, 1, 3, 4), (10, 0.25, 27, 2, 5, 2),
                                                 (9, 0.4, 125, 1, 2, 3), (6, 0.5, 1, 1, 4, 6)])
def test_wgrad_matches_conv3d_autograd(G, density, K, d, Ci, Co):
    rng = np.random.default_rng(43 + G + K + d)
    coords = random_sites(rng, G, density)
    N = coords.shape[0]
    feats = rng.standard_normal((N, Ci)).astype(np.float32)
    dout = rng.standard_normal((N, Co)).astype(np.float32)
    nb = oracle.nmap(coords, K, d)
    got, sab = oracle.wgrad(feats, dout, nb)
    ref = dense_conv_weight_grad(coords, feats, dout, K, d, Co)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11 * (1 + np.abs(ref).max()))
    assert (sab >= np.abs(got) - 1e-12).all()


def test_wgrad_contraction_identity_and_k1():
    rng = np.random.default_rng(47)
    coords = random_sites(rng, 14, 0.2)
    N, K, Ci, Co = coords.shape[0], 27, 6, 5
    feats = rng.standard_normal((N, Ci)).astype(np.float32)
    dout = rng.standard_normal((N, Co)).astype(np.float32)
    W = rng.standard_normal((K, Ci, Co)).astype(np.float32)
    nb = oracle.nmap(coords, K, 1)
    dw = oracle.wgrad(feats, dout, nb, with_abs=False)
    lhs = float((dw * W.astype(np.float64)).sum())
    rhs = float((oracle.forward(feats, nb, W, None, with_abs=False) * dout.astype(np.float64)).sum())
    assert abs(lhs - rhs) <= 1e-11 * (abs(lhs) + 1.0)
    nb1 = oracle.nmap(coords, 1, 1)
    dw1 = oracle.wgrad(feats, dout, nb1, with_abs=False)
    np.testing.assert_allclose(dw1[0], feats.astype(np.float64).T @ dout.astype(np.float64), rtol=1e-13, atol=1e-12)


# --- mixed dtypes: the cast of feats to w's dtype --------------------------

def _f32_bits(bits):
    return torch.from_numpy(np.array(bits, dtype=np.uint32).view(np.float32))


def _bf16_bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


# (float32 bits, bfloat16 bits) worked out by hand: t = top 16 bits, the
# halfway point between t and t + 1 is t's bits followed by 0x8000.
CAST_CASES = [
    (0x3F808000, 0x3F80),   # 1 + 2^-8: tie, t = 0x3F80 even -> stays
    (0x3F818000, 0x3F82),   # 1 + 3*2^-8: tie, t = 0x3F81 odd -> up
    (0x3F808001, 0x3F81),   # just above half -> up
    (0x3F807FFF, 0x3F80),   # just below half -> down
    (0xBF818000, 0xBF82),   # negative tie: magnitude rounds to even
    (0x7F7F7FFF, 0x7F7F),   # below half past the largest finite -> largest finite
    (0x7F7F8000, 0x7F80),   # tie past the largest finite (odd) -> overflow to +inf
    (0x7F7FFFFF, 0x7F80),   # float32 max -> +inf
    (0xFF7FFFFF, 0xFF80),   # -float32 max -> -inf
    (0x00008000, 0x0000),   # subnormal tie, even -> 0
    (0x00018000, 0x0002),   # subnormal tie, odd -> up
    (0x007FFFFF, 0x0080),   # largest subnormal rounds up to the smallest normal
    (0x7F800000, 0x7F80),   # +inf
    (0xFF800000, 0xFF80),   # -inf
    (0x80000000, 0x8000),   # -0
    (0x00000000, 0x0000),   # +0
    (0x7FC00001, 0x7FC0),   # quiet NaN
    (0x7F800001, 0x7FC0),   # signalling NaN -> quiet NaN
    (0xFF800001, 0xFFC0),   # negative NaN keeps its sign
]


def test_cast_f32_to_bf16_handworked():
    src = _f32_bits([a for a, _ in CAST_CASES])
    got = _bf16_bits(oracle.cast(src, torch.bfloat16))
    assert [int(v) for v in got] == [b for _, b in CAST_CASES]


def test_cast_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(77)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    ties = (bits & 0xFFFF0000) | 0x8000                  # exact halfway points
    near = (bits & 0xFFFF0000) | rng.choice([0x7FFF, 0x8001, 0x0001, 0xFFFF], bits.size).astype(np.uint32)
    allb = np.concatenate([bits, ties, near])
    x = _f32_bits(allb)
    got = _bf16_bits(oracle.cast(x, torch.bfloat16))
    ref = _bf16_bits(x.to(torch.bfloat16))
    nan = np.isnan(x.numpy())
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN payloads are not specified; NaN must stay NaN with its sign
    g = torch.from_numpy(got[nan].view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.isnan(g).all()
    assert np.array_equal(got[nan] >> 15, (allb[nan] >> 31).astype(np.uint16))


def test_cast_bf16_to_f32_all_patterns():
    b = torch.from_numpy(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    got = oracle.cast(b, torch.float32).numpy().view(np.uint32)
    assert np.array_equal(got, np.arange(1 << 16, dtype=np.uint32) << 16)
    # round trip through the other direction is the identity
    assert np.array_equal(_bf16_bits(oracle.cast(oracle.cast(b, torch.float32), torch.bfloat16))[:0x7F81],
                          np.arange(0x7F81, dtype=np.uint16))


def test_forward_mixed_k1_identity_is_the_cast():
    rng = np.random.default_rng(78)
    N, C = 40, 32
    bits = rng.integers(0, 2 ** 32, size=N * C, dtype=np.uint64).astype(np.uint32)
    bits = (bits & 0x807FFFFF) | (rng.integers(100, 150, N * C, dtype=np.uint32) << 23)   # normal, moderate
    bits[::3] = (bits[::3] & 0xFFFF0000) | 0x8000                                          # ties
    feats = _f32_bits(bits).reshape(N, C)
    w = torch.eye(C).reshape(1, C, C).to(torch.bfloat16)
    nbr = np.arange(N, dtype=np.int32).reshape(1, N)
    out = oracle.forward_mixed(feats, nbr, w, with_abs=False)
    assert np.array_equal(out, feats.to(torch.bfloat16).double().numpy())


def test_forward_mixed_reduces_to_same_dtype_forward():
    rng = np.random.default_rng(79)
    coords = np.argwhere(rng.random((7, 7, 7)) < 0.4).astype(np.int32)
    N, K = coords.shape[0], 27
    nb = oracle.nmap(coords, K, 1)
    fb = torch.from_numpy(rng.standard_normal((N, 32)).astype(np.float32)).to(torch.bfloat16)
    wb = torch.from_numpy(rng.standard_normal((K, 32, 64)).astype(np.float32)).to(torch.bfloat16)
    bias = torch.from_numpy(rng.standard_normal(64).astype(np.float32))
    # fp32 feats that are bf16 values: the cast changes nothing
    a, sa = oracle.forward_mixed(fb.float(), nb, wb, bias)
    b, sb = oracle.forward(fb, nb, wb, bias)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)
    # bf16 feats with fp32 weights: widening is exact
    wf = torch.from_numpy(rng.standard_normal((K, 32, 64)).astype(np.float32))
    a, _ = oracle.forward_mixed(fb, nb, wf, bias)
    b, _ = oracle.forward(fb.float(), nb, wf, bias)
    assert np.array_equal(a, b)
