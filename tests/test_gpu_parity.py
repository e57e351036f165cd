"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Neighbour maps are compared bit for bit (full maps, every workload).  Forward
outputs are compared with oracle/compare.py's tolerances: every output row on
the small workloads, sampled rows (random rows plus whole schedule tiles,
including the ragged last one) on the large ones, in the launch
configuration the benchmark times.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.compare import check_forward
import submanifold_sparse_convolution_spconv_amd as sp

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


_cache = {}


def workload(name):
    if name not in _cache:
        wl = W.by_name(name)
        coords = W.geometry(wl)
        feats, w, bias = W.values(wl, coords.shape[0])
        _cache.clear()                      # keep one workload resident
        _cache[name] = (wl, coords, feats, w, bias)
    return _cache[name]


def dtype_name(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def gpu_build(coords, K, d):
    return sp.spconv_build_nmap(torch.from_numpy(np.ascontiguousarray(coords)).to(DEV), K, d)


def check_rows(feats, nb_cols, w, bias, gpu_rows, tag):
    ref, S = oracle.forward(feats, nb_cols, w, bias)
    rep = check_forward(gpu_rows, ref, S, None if bias is None else bias.numpy(), dtype_name(w))
    say(tag, rep)
    assert rep["fail"] == 0, rep
    return rep


ALL = ["uniform32", "shell64", "surf256", "surf512d2", "surf1024"]


@pytest.mark.parametrize("name", ALL)
def test_nmap_bit_exact(name):
    wl, coords, *_ = workload(name)
    N = coords.shape[0]
    say(f"[nmap] {name} N={N} K={wl.K} dilation={wl.dilation}")
    nm = gpu_build(coords, wl.K, wl.dilation)
    nbr, order = nm.export()
    torch.cuda.synchronize()
    g = nbr.cpu().numpy()
    ref = oracle.nmap(coords, wl.K, wl.dilation)
    assert g.shape == ref.shape
    mism = int((g != ref).sum())
    say(f"[nmap] {name} mismatches={mism} valid_pairs={nm.valid_pairs}")
    assert mism == 0
    assert nm.valid_pairs == int((ref != N).sum())
    # schedule: a permutation whose 128-row half tiles hold consecutive Morton
    # ranks, each sorted by the rows' validity masks
    o = order.cpu().numpy().astype(np.int64)
    assert np.array_equal(np.sort(o), np.arange(N))
    rank = np.empty(N, np.int64)
    rank[np.argsort(oracle.morton(coords), kind="stable")] = np.arange(N)
    half_of_row = np.arange(N) // 128
    assert np.array_equal(rank[o] // 128, half_of_row)
    valid = (ref[:, o] != N)
    keys = (valid[:min(wl.K, 63)].astype(np.uint64) << np.arange(min(wl.K, 63), dtype=np.uint64)[:, None]).sum(0)
    for t0 in range(0, N, 128):
        kk = keys[t0:t0 + 128]
        assert (np.diff(kk.astype(np.float64)) >= 0).all(), t0
    del nm


@pytest.mark.parametrize("name", ["uniform32", "shell64"])
def test_forward_full(name):
    wl, coords, feats, w, bias = workload(name)
    N = coords.shape[0]
    say(f"[fwd-full] {name} N={N} Ci={wl.Ci} Co={wl.Co} {wl.dtype}")
    nm = gpu_build(coords, wl.K, wl.dilation)
    out = sp.spconv_forward(feats.to(DEV), nm, w.to(DEV), bias.to(DEV))
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    nb = oracle.nmap(coords, wl.K, wl.dilation)
    check_rows(feats, nb, w, bias, g, f"[fwd-full] {name}")


ROW_BLOCK = 1 << 20


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["surf256", "surf512d2", "surf1024"])
def test_forward_every_row_full_size(name):
    """Every output of the full-size workloads, for the unpacked forward and
    the packed one the benchmark times, against the oracle streamed over
    blocks of caller rows."""
    wl, coords, feats, w, bias = workload(name)
    N = coords.shape[0]
    say(f"[fwd-every-row] {name} N={N} Ci={wl.Ci} Co={wl.Co} {wl.dtype}")
    nm = gpu_build(coords, wl.K, wl.dilation)
    fd, wd, bd = feats.to(DEV), w.to(DEV), bias.to(DEV)
    outs = {"forward": sp.spconv_forward(fd, nm, wd, bd)}
    wp = sp.spconv_pack_weights(wd)
    if wp.numel():
        outs["forward_packed"] = sp.spconv_forward_packed(fd, nm, wd, wp, bd)
    torch.cuda.synchronize()
    del fd
    host = {k: v.float().cpu().numpy() for k, v in outs.items()}
    del outs
    nb = oracle.nmap(coords, wl.K, wl.dilation)
    say(f"[fwd-every-row] {name} oracle map done; {len(host)} GPU outputs to check")
    worst = {}
    for r0 in range(0, N, ROW_BLOCK):
        r1 = min(N, r0 + ROW_BLOCK)
        ref, S = oracle.forward(feats, np.ascontiguousarray(nb[:, r0:r1]), w, bias)
        for kind, g in host.items():
            rep = check_forward(g[r0:r1], ref, S, bias.numpy(), wl.dtype)
            assert rep["fail"] == 0, (kind, r0, rep)
            worst[kind] = max(worst.get(kind, 0.0), rep["max_norm_err"])
        say(f"[fwd-every-row] {name} rows {r0}..{r1} ok " + str({k: f"{v:.2e}" for k, v in worst.items()}))


def random_sites(rng, G, density, origin=(0, 0, 0)):
    m = rng.random((G, G, G)) < density
    c = np.argwhere(m).astype(np.int64) + np.array(origin)
    return c[rng.permutation(c.shape[0])].astype(np.int32)


SMALL = [
    # G, density, K, d, Ci, Co, dtype
    (10, 0.3, 27, 1, 32, 32, "f32"),
    (12, 0.2, 27, 2, 64, 96, "f32"),
    (9, 0.5, 125, 1, 32, 64, "bf16"),
    (16, 0.08, 27, 3, 128, 64, "bf16"),
    (14, 0.15, 1, 1, 128, 128, "bf16"),
    (11, 0.4, 27, 1, 256, 32, "bf16"),
    (8, 0.6, 27, 1, 256, 64, "f32"),
    (13, 0.3, 27, 1, 128, 256, "f32"),
    (3, 0.5, 27, 1, 32, 32, "bf16"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "G%d_K%d_d%d_%dx%d_%s" % (c[0], c[2], c[3], c[4], c[5], c[6]))
def test_small_grids(case):
    G, dens, K, d, Ci, Co, dt = case
    rng = np.random.default_rng(G * 7 + K + d + Ci + Co)
    coords = random_sites(rng, G, dens, origin=(-5, 3, 100))
    N = coords.shape[0]
    say(f"[small] N={N} K={K} d={d} Ci={Ci} Co={Co} {dt}")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    feats = torch.from_numpy(rng.standard_normal((N, Ci)).astype(np.float32)).to(tdt)
    w = torch.from_numpy((rng.standard_normal((K, Ci, Co)) / np.sqrt(K * Ci)).astype(np.float32)).to(tdt)
    bias = torch.from_numpy(rng.standard_normal(Co).astype(np.float32))
    nm = gpu_build(coords, K, d)
    nbr, _ = nm.export()
    out = sp.spconv_forward(feats.to(DEV), nm, w.to(DEV), bias.to(DEV))
    torch.cuda.synchronize()
    ref_nb = oracle.nmap(coords, K, d)
    assert np.array_equal(nbr.cpu().numpy(), ref_nb)
    check_rows(feats, ref_nb, w, bias, out.float().cpu().numpy(), "[small]")


# fp32 maps of 16,384 to 65,536 rows take 2 or 4 16-row blocks per workgroup
# in the offset-split kernel (enough workgroups for two per CU on 256 CUs)
@pytest.mark.parametrize("G, Ci, Co", [(40, 32, 64), (48, 32, 32), (48, 64, 64)],
                         ids=["two_blocks_32x64", "four_blocks_32x32", "two_blocks_64x64"])
def test_split_block_counts(G, Ci, Co):
    rng = np.random.default_rng(G + Ci + Co)
    coords = random_sites(rng, G, 0.35, origin=(7, -20, 3))
    N = coords.shape[0]
    assert 16384 <= N <= 65536
    say(f"[split] N={N} Ci={Ci} Co={Co} f32")
    feats = torch.from_numpy(rng.standard_normal((N, Ci)).astype(np.float32))
    w = torch.from_numpy((rng.standard_normal((27, Ci, Co)) / np.sqrt(27 * Ci)).astype(np.float32))
    bias = torch.from_numpy(rng.standard_normal(Co).astype(np.float32))
    nm = gpu_build(coords, 27, 1)
    nbr, _ = nm.export()
    out = sp.spconv_forward(feats.to(DEV), nm, w.to(DEV), bias.to(DEV))
    torch.cuda.synchronize()
    ref_nb = oracle.nmap(coords, 27, 1)
    assert np.array_equal(nbr.cpu().numpy(), ref_nb)
    check_rows(feats, ref_nb, w, bias, out.cpu().numpy(), "[split]")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_all_sentinel_returns_bias(dt):
    rng = np.random.default_rng(5)
    N, K, Ci, Co = 700, 27, 64, 64
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    feats = torch.from_numpy(rng.standard_normal((N, Ci)).astype(np.float32)).to(tdt).to(DEV)
    w = torch.from_numpy(rng.standard_normal((K, Ci, Co)).astype(np.float32)).to(tdt).to(DEV)
    bias = torch.from_numpy(rng.standard_normal(Co).astype(np.float32)).to(DEV)
    for fill in (N, -1, N + 12345):
        say(f"[sentinel] {dt} fill={fill}")
        nm = sp.spconv_nmap_wrap(torch.full((K, N), fill, dtype=torch.int32, device=DEV))
        out = sp.spconv_forward(feats, nm, w, bias)
        assert torch.equal(out, bias.to(tdt)[None, :].expand(N, Co))
        assert nm.valid_pairs == 0
        out0 = sp.spconv_forward(feats, nm, w, None)
        assert torch.equal(out0, torch.zeros_like(out0))
        assert not torch.signbit(out0.float()).any()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_k1_is_gemm(dt):
    rng = np.random.default_rng(6)
    coords = random_sites(rng, 40, 0.02)
    N, Ci, Co = coords.shape[0], 128, 128
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    feats = torch.from_numpy(rng.standard_normal((N, Ci)).astype(np.float32)).to(tdt)
    w = torch.from_numpy((rng.standard_normal((1, Ci, Co)) / np.sqrt(Ci)).astype(np.float32)).to(tdt)
    bias = torch.from_numpy(rng.standard_normal(Co).astype(np.float32))
    say(f"[k1] N={N} {dt}")
    nm = gpu_build(coords, 1, 1)
    out = sp.spconv_forward(feats.to(DEV), nm, w.to(DEV), bias.to(DEV)).float().cpu().numpy()
    ref = feats.double().numpy() @ w[0].double().numpy() + bias.double().numpy()
    S = np.abs(feats.double().numpy()) @ np.abs(w[0].double().numpy())
    rep = check_forward(out, ref, S, bias.numpy(), dt)
    say("[k1]", rep)
    assert rep["fail"] == 0


def test_ones_closed_form():
    rng = np.random.default_rng(7)
    coords = random_sites(rng, 20, 0.25)
    N, Ci, Co = coords.shape[0], 32, 64
    bias = torch.arange(Co, dtype=torch.float32) * 0.5
    nm = gpu_build(coords, 27, 1)
    nbr, _ = nm.export()
    v = (nbr != N).sum(0).cpu().double()
    for tdt in (torch.float32, torch.bfloat16):
        say(f"[ones] {tdt}")
        out = sp.spconv_forward(torch.ones((N, Ci), dtype=tdt, device=DEV), nm,
                                torch.ones((27, Ci, Co), dtype=tdt, device=DEV), bias.to(DEV))
        ref = (bias.double()[None, :] + Ci * v[:, None]).to(tdt)
        assert torch.equal(out.cpu(), ref)


def test_determinism_shuffle_and_wrap():
    wl, coords, feats, w, bias = workload("shell64")
    N = coords.shape[0]
    fd, wd, bd = feats.to(DEV), w.to(DEV), bias.to(DEV)
    say("[determinism] shell64")
    nm = gpu_build(coords, 27, 1)
    o1 = sp.spconv_forward(fd, nm, wd, bd)
    o2 = sp.spconv_forward(fd, nm, wd, bd)
    assert torch.equal(o1, o2)
    # a different caller order: same map after relabelling, same outputs
    perm = np.random.default_rng(99).permutation(N)
    nm2 = gpu_build(coords[perm], 27, 1)
    o3 = sp.spconv_forward(fd[torch.from_numpy(perm).to(DEV)], nm2, wd, bd)
    assert torch.equal(o3, o1[torch.from_numpy(perm).to(DEV)])
    nb1, _ = nm.export()
    nb2, _ = nm2.export()
    inv = np.empty(N, np.int64)
    inv[perm] = np.arange(N)
    a = nb1.cpu().numpy()[:, perm]
    b = nb2.cpu().numpy()
    b_relab = np.where(b == N, N, perm[np.minimum(b, N - 1)])
    assert np.array_equal(a, b_relab)
    # the page's interface: a caller-made map, with an N+1-row padded feats
    nm3 = sp.spconv_nmap_wrap(nb1)
    padded = torch.cat([fd, torch.zeros((1, fd.shape[1]), dtype=fd.dtype, device=DEV)])
    o4 = sp.spconv_forward(padded, nm3, wd, bd)
    assert torch.equal(o4, o1)


@pytest.mark.parametrize("G, dens", [(48, 0.7), (24, 0.5)], ids=["f32_gather", "f32_split"])
def test_f32_caller_order_independent(G, dens):
    # fp32 maps above 65,536 rows run the gather kernel, smaller ones the
    # offset-split kernel: either way each output adds its terms in a fixed
    # order, so the same cloud in another caller order gives the same rows
    rng = np.random.default_rng(G)
    coords = random_sites(rng, G, dens, origin=(-30, 2, 9))
    N = coords.shape[0]
    say(f"[f32 order] N={N}")
    feats = torch.from_numpy(rng.standard_normal((N, 32)).astype(np.float32)).to(DEV)
    w = torch.from_numpy((rng.standard_normal((27, 32, 64)) / 30).astype(np.float32)).to(DEV)
    bias = torch.from_numpy(rng.standard_normal(64).astype(np.float32)).to(DEV)
    o1 = sp.spconv_forward(feats, gpu_build(coords, 27, 1), w, bias)
    perm = np.random.default_rng(G + 1).permutation(N)
    pd = torch.from_numpy(perm).to(DEV)
    o2 = sp.spconv_forward(feats[pd], gpu_build(coords[perm], 27, 1), w, bias)
    assert torch.equal(o2, o1[pd])


def test_build_errors():
    say("[errors]")
    dup = torch.tensor([[0, 0, 0], [5, 5, 5], [0, 0, 0]], dtype=torch.int32, device=DEV)
    with pytest.raises(sp.SpconvError) as e:
        sp.spconv_build_nmap(dup)
    assert e.value.code == -4
    far = torch.tensor([[0, 0, 0], [1 << 20, 0, 0]], dtype=torch.int32, device=DEV)
    with pytest.raises(sp.SpconvError) as e:
        sp.spconv_build_nmap(far)
    assert e.value.code == -3
    neg = torch.tensor([[-(1 << 20), 0, 0], [(1 << 20) - 1, 7, 7]], dtype=torch.int32, device=DEV)
    nm = sp.spconv_build_nmap(neg)
    nbr, _ = nm.export()
    assert nbr[13].tolist() == [0, 1] and int((nbr != 2).sum()) == 2


def test_tiny_and_ragged():
    for N in (1, 2, 255, 256, 257, 1000):
        rng = np.random.default_rng(N)
        lin = rng.choice(64 ** 3, N, replace=False)
        coords = np.stack([lin // 4096, (lin // 64) % 64, lin % 64], 1).astype(np.int32)
        say(f"[ragged] N={N}")
        feats = torch.from_numpy(rng.standard_normal((N, 32)).astype(np.float32))
        w = torch.from_numpy(rng.standard_normal((27, 32, 32)).astype(np.float32) / 30)
        bias = torch.from_numpy(rng.standard_normal(32).astype(np.float32))
        nm = gpu_build(coords, 27, 1)
        nbr, _ = nm.export()
        out = sp.spconv_forward(feats.to(DEV), nm, w.to(DEV), bias.to(DEV))
        torch.cuda.synchronize()
        ref_nb = oracle.nmap(coords, 27, 1)
        assert np.array_equal(nbr.cpu().numpy(), ref_nb)
        check_rows(feats, ref_nb, w, bias, out.cpu().numpy(), f"[ragged] N={N}")


def test_even_lattice_dilation2():
    # every coordinate even: all voxels share the same low coordinate bits,
    # the case a brick-local hash has to spread out
    rng = np.random.default_rng(21)
    coords = (random_sites(rng, 30, 0.3).astype(np.int64) * 2 - 17 * 2).astype(np.int32)
    N = coords.shape[0]
    say(f"[lattice] N={N}")
    feats = torch.from_numpy(rng.standard_normal((N, 64)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((27, 64, 64)) / 40).astype(np.float32)).to(torch.bfloat16)
    bias = torch.from_numpy(rng.standard_normal(64).astype(np.float32))
    for d in (1, 2):
        nm = gpu_build(coords, 27, d)
        nbr, _ = nm.export()
        out = sp.spconv_forward(feats.to(DEV), nm, w.to(DEV), bias.to(DEV))
        torch.cuda.synchronize()
        ref_nb = oracle.nmap(coords, 27, d)
        assert np.array_equal(nbr.cpu().numpy(), ref_nb)
        assert nm.valid_pairs == int((ref_nb != N).sum())
        check_rows(feats, ref_nb, w, bias, out.float().cpu().numpy(), f"[lattice] d={d}")


def query_paths(coords, d):
    """Which of the tile query's paths each 256-row tile of the Morton schedule
    takes for the 3x3x3 stencil at dilation d: 'hashed' (the tile's distinct
    bricks fit the 512-slot LDS set) or 'per-row' (more distinct bricks than
    slots: the set overflows and every row probes the global table).  Between
    256 and 512 distinct bricks either path may run; those tiles are 'either'."""
    u = coords.astype(np.int64) + (1 << 20)
    o = np.argsort(oracle.morton(coords), kind="stable")
    paths = []
    for t0 in range(0, len(o), 256):
        uu = u[o[t0:t0 + 256]]
        lo = np.where(uu >= d, uu - d, uu) >> 2
        hi = np.where(uu + d < (1 << 21), uu + d, uu) >> 2
        keys = set()
        for i in range(8):
            b = np.stack([hi[:, 0] if i & 4 else lo[:, 0], hi[:, 1] if i & 2 else lo[:, 1],
                          hi[:, 2] if i & 1 else lo[:, 2]], 1)
            keys.update(map(tuple, b))
        paths.append("per-row" if len(keys) > 512 else "hashed" if len(keys) <= 256 else "either")
    return paths


def check_schedule(nm, ref, K):
    N = ref.shape[1]
    _, order = nm.export()
    o = order.cpu().numpy().astype(np.int64)
    assert np.array_equal(np.sort(o), np.arange(N))
    valid = ref[:, o] != N
    keys = (valid[:min(K, 63)].astype(np.uint64) << np.arange(min(K, 63), dtype=np.uint64)[:, None]).sum(0)
    for t0 in range(0, N, 128):
        assert (np.diff(keys[t0:t0 + 128].astype(np.float64)) >= 0).all(), t0


def test_query_paths():
    rng = np.random.default_rng(31)
    dense = np.argwhere(np.ones((24, 24, 24), bool)).astype(np.int32) - 7
    sparse = np.unique(rng.integers(-(1 << 19), 1 << 19, (20000, 3)), axis=0).astype(np.int32)
    mixed = np.unique(np.concatenate([dense, sparse[:3000], random_sites(rng, 40, 0.05, origin=(300, 0, 0))]),
                      axis=0).astype(np.int32)
    cases = [("dense", dense, {"hashed"}), ("sparse", sparse, {"per-row"}), ("mixed", mixed, {"hashed", "per-row"})]
    for name, coords, want in cases:
        coords = coords[rng.permutation(coords.shape[0])]
        N = coords.shape[0]
        for d in (1, 2):
            paths = query_paths(coords, d)
            say(f"[paths] {name} N={N} d={d} tiles: " +
                ", ".join(f"{p}={paths.count(p)}" for p in ("hashed", "either", "per-row")))
            assert want <= set(paths)
            nm = gpu_build(coords, 27, d)
            nbr, _ = nm.export()
            torch.cuda.synchronize()
            ref = oracle.nmap(coords, 27, d)
            assert np.array_equal(nbr.cpu().numpy(), ref)
            assert nm.valid_pairs == int((ref != N).sum())
            check_schedule(nm, ref, 27)
