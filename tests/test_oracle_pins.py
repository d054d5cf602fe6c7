"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formula: each compares the oracle with an
independent route (brute force, a special case with a closed form, a
mathematical identity, a number printed on the pages).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import bf16, compare, decompose, forward, sizes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_values(rng, shape, std=1.0):
    return bf16.round_bf16(rng.standard_normal(shape) * std)


# --------------------------------------------------------------------------
# bfloat16 rounding
# --------------------------------------------------------------------------
@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                 # tie, mantissa 0 is even
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie, rounds up to the even mantissa 2
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),    # just above the tie
    (-2.5, 0xC020),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (2.0 ** -130, 0x0008),                     # subnormal
    (3.4e38, 0x7F80),                          # rounds past the bf16 maximum
    (3.3895313892515355e38, 0x7F7F),           # bf16 maximum itself
])
def test_bf16_bit_patterns(value, bits):
    assert int(bf16.bits_bf16(np.array([value]))[0]) == bits


def test_bf16_matches_torch_rounding():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    a = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000),
                        rng.standard_normal(1000)])
    ours = bf16.bits_bf16(a)
    t = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, t)


# --------------------------------------------------------------------------
# forward: special cases with closed forms, and the factored/explicit identity
# --------------------------------------------------------------------------
def test_identity_block_scales_input():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 6))
    s = np.array([2.0, -1.0, 0.5, 3.0, 1.0, 0.0])
    y = forward.factored(x, np.eye(6), s, np.zeros((6, 0)), np.zeros((6, 0)))
    assert np.array_equal(y, x * s[None, :])


def test_rank_one_delta_closed_form():
    # W0 = 0: y[t, i] = u_i * (sum_j v_j x[t, j]); N != K so a transposed V fails
    rng = np.random.default_rng(2)
    T, N, K = 2, 3, 5
    x = rng.standard_normal((T, K))
    u = rng.standard_normal(N)
    v = rng.standard_normal(K)
    y = forward.factored(x, np.zeros((N, K)), np.ones(N), u[:, None], v[:, None])
    for t in range(T):
        dot = sum(v[j] * x[t, j] for j in range(K))
        for i in range(N):
            assert abs(y[t, i] - u[i] * dot) <= 1e-14 * (1 + abs(u[i] * dot))


def test_forward_brute_force_loops():
    rng = np.random.default_rng(3)
    T, N, K, r = 2, 4, 5, 3
    x, W0 = rng.standard_normal((T, K)), rng.standard_normal((N, K))
    s, U, V = rng.standard_normal(N), rng.standard_normal((N, r)), rng.standard_normal((K, r))
    y = forward.factored(x, W0, s, U, V)
    for t in range(T):
        for i in range(N):
            acc = 0.0
            for j in range(K):
                w = s[i] * W0[i, j]
                for k in range(r):
                    w += U[i, k] * V[j, k]
                acc += w * x[t, j]
            assert abs(y[t, i] - acc) <= 1e-12 * (1 + abs(acc))


@pytest.mark.parametrize("T,N,K,r", [(1, 64, 48, 4), (4, 300, 200, 32), (7, 96, 512, 96)])
def test_factored_equals_explicit(T, N, K, r):
    """P2: the factored forward is the same map as the explicit effective
    weight; the two differ only by rounding order (fp64)."""
    rng = np.random.default_rng(T * 1000 + N)
    x = bf16_values(rng, (T, K))
    W0 = bf16_values(rng, (N, K), 1 / math.sqrt(K))
    s = rng.normal(1, 0.05, N).astype(np.float32).astype(np.float64)
    U, V = bf16_values(rng, (N, r), 0.02), bf16_values(rng, (K, r), 0.02)
    yf = forward.factored(x, W0, s, U, V)
    ye = forward.explicit(x, W0, s, U, V)
    scale = np.abs(x) @ (np.abs(s)[:, None] * np.abs(W0) + np.abs(U) @ np.abs(V).T).T
    assert np.all(np.abs(yf - ye) <= 1e-12 * scale + 1e-300)


def test_stacked_is_concatenation_and_tied_slot():
    """P7 + P8: a stacked call is its children's outputs side by side; a tied
    child repeats the previous child's output exactly."""
    rng = np.random.default_rng(4)
    K = 40
    x = bf16_values(rng, (3, K))
    ch = []
    for n in (24, 8, 8):
        ch.append((bf16_values(rng, (n, K)), rng.normal(1, .05, n), bf16_values(rng, (n, 4)),
                   bf16_values(rng, (K, 4))))
    y = forward.stacked(x, ch)
    assert np.array_equal(y[:, :24], forward.factored(x, *ch[0]))
    assert np.array_equal(y[:, 24:32], forward.factored(x, *ch[1]))
    assert np.array_equal(y[:, 32:], forward.factored(x, *ch[2]))
    yt = forward.stacked(x, [ch[0], ch[1], "dup"])
    assert np.array_equal(yt[:, 24:32], yt[:, 32:40])


# --------------------------------------------------------------------------
# decomposition
# --------------------------------------------------------------------------
def test_band_assignment():
    assert [decompose.band_of(l, 26, 13) for l in range(6)] == [0, 0, 1, 1, 2, 2]
    # Gemma 4: "5 bands (12 layers per band)" over 60 layers
    counts = np.bincount([decompose.band_of(l, 60, 5) for l in range(60)])
    assert list(counts) == [12] * 5
    assert [decompose.band_of(l, 26, 26) for l in range(26)] == list(range(26))
    assert {decompose.band_of(l, 26, 1) for l in range(26)} == {0}
    # every band of an uneven split is contiguous and non-empty
    b = [decompose.band_of(l, 7, 3) for l in range(7)]
    assert b == sorted(b) and set(b) == {0, 1, 2}


@pytest.mark.parametrize("rank", [1, 4, 32])
def test_passthrough_is_exact(rank):
    """P1: with one layer per band the decomposition returns the layer's own
    weight, s = 1 and a zero delta, exactly; the factored forward then equals
    the dense product bit for bit."""
    rng = np.random.default_rng(rank)
    L, N, K = 4, 48, 40
    Ws = [bf16_values(rng, (N, K), 1 / math.sqrt(K)) for _ in range(L)]
    res = decompose.decompose_family(Ws, num_bands=L, rank=rank, store=True)
    x = bf16_values(rng, (5, K))
    for l in range(L):
        assert np.array_equal(res["W0"][l], Ws[l])
        assert np.all(res["s"][l] == 1.0)
        assert np.all(res["U"][l] @ res["V"][l].T == 0.0)
        assert res["err"][l] == 0.0
        y = forward.factored(x, res["W0"][l], res["s"][l], res["U"][l], res["V"][l])
        assert np.array_equal(y, forward.dense(x, Ws[l]))


@pytest.mark.parametrize("G", [1, 2, 3])
def test_full_rank_reconstructs(G):
    """P3: a rank of min(N, K) leaves no residual, whatever the sharing."""
    rng = np.random.default_rng(10 + G)
    L, N, K = 6, 20, 12
    Ws = [rng.standard_normal((N, K)) for _ in range(L)]
    res = decompose.decompose_family(Ws, num_bands=G, rank=min(N, K), store=False)
    assert max(res["err"]) <= 1e-12
    # rank above full rank is clamped to min(N, K)
    res2 = decompose.decompose_family(Ws, num_bands=G, rank=100, store=False)
    assert all(u.shape[1] == min(N, K) for u in res2["U"])


@pytest.mark.parametrize("rank", [1, 5, 16])
def test_eckart_young_tail_energy(rank):
    """P4: the reconstructed error equals the discarded singular-value energy
    of the residual (unrounded decomposition)."""
    rng = np.random.default_rng(20 + rank)
    L, N, K = 4, 40, 24
    Ws = [rng.standard_normal((N, K)) / math.sqrt(K) for _ in range(L)]
    res = decompose.decompose_family(Ws, num_bands=2, rank=rank, store=False)
    for l in range(L):
        ey = decompose.eckart_young_error(Ws[l], res["sigma"][l], rank)
        assert abs(ey - res["err"][l]) <= 1e-10


# ---- P5: brute force on tiny inputs -------------------------------------
def _jacobi_eigh(A, sweeps=60):
    """Cyclic Jacobi eigen-solver for a small symmetric matrix (pure Python
    loops; shares nothing with LAPACK)."""
    n = len(A)
    a = [[float(A[i][j]) for j in range(n)] for i in range(n)]
    v = [[1.0 if i == j else 0.0 for j in range(n)] for i in range(n)]
    for _ in range(sweeps):
        off = sum(a[i][j] ** 2 for i in range(n) for j in range(n) if i != j)
        if off < 1e-300:
            break
        for p in range(n):
            for q in range(p + 1, n):
                if abs(a[p][q]) < 1e-300:
                    continue
                theta = (a[q][q] - a[p][p]) / (2.0 * a[p][q])
                t = (1.0 if theta >= 0 else -1.0) / (abs(theta) + math.sqrt(theta * theta + 1.0))
                c = 1.0 / math.sqrt(t * t + 1.0)
                s = t * c
                for k in range(n):
                    akp, akq = a[k][p], a[k][q]
                    a[k][p], a[k][q] = c * akp - s * akq, s * akp + c * akq
                for k in range(n):
                    apk, aqk = a[p][k], a[q][k]
                    a[p][k], a[q][k] = c * apk - s * aqk, s * apk + c * aqk
                for k in range(n):
                    vkp, vkq = v[k][p], v[k][q]
                    v[k][p], v[k][q] = c * vkp - s * vkq, s * vkp + c * vkq
    return [a[i][i] for i in range(n)], v


def _brute_decompose(Ws, G, rank):
    """Band means by loops, s by bisection on the slope of the row error, the rank-r
    residual approximation from a Jacobi eigen-decomposition of R^T R."""
    L = len(Ws)
    N, K = len(Ws[0]), len(Ws[0][0])
    errs, uvs = [], []
    for l in range(L):
        b = (l * G) // L
        members = [m for m in range(L) if (m * G) // L == b]
        W0 = [[sum(Ws[m][i][j] for m in members) / len(members) for j in range(K)] for i in range(N)]
        W = Ws[l]
        s = []
        for i in range(N):
            # the row error is a convex quadratic in c; bisect on the sign of
            # its slope, -2 * sum_j W0[i][j] * (W[i][j] - c * W0[i][j])
            slope = lambda c: -sum(W0[i][j] * (W[i][j] - c * W0[i][j]) for j in range(K))
            lo, hi = -50.0, 50.0
            for _ in range(200):
                mid = 0.5 * (lo + hi)
                if slope(mid) > 0:
                    hi = mid
                else:
                    lo = mid
            s.append(0.5 * (lo + hi))
        R = [[W[i][j] - s[i] * W0[i][j] for j in range(K)] for i in range(N)]
        RtR = [[sum(R[i][p] * R[i][q] for i in range(N)) for q in range(K)] for p in range(K)]
        lam, vec = _jacobi_eigh(RtR)
        order = sorted(range(K), key=lambda k: -lam[k])[:min(rank, N, K)]
        # rank-r approximation R Q_r Q_r^T
        UVt = [[sum(R[i][m] * sum(vec[m][k] * vec[j][k] for k in order) for m in range(K))
                for j in range(K)] for i in range(N)]
        rec = [[s[i] * W0[i][j] + UVt[i][j] for j in range(K)] for i in range(N)]
        num = math.sqrt(sum((W[i][j] - rec[i][j]) ** 2 for i in range(N) for j in range(K)))
        den = math.sqrt(sum(W[i][j] ** 2 for i in range(N) for j in range(K)))
        errs.append(num / den)
        srt = sorted(lam, reverse=True)
        gap = min(rank, N, K) < K and srt[min(rank, N, K) - 1] > srt[min(rank, N, K)] * (1 + 1e-6)
        uvs.append((np.array(UVt), gap))
    return errs, uvs


@pytest.mark.parametrize("L,G,N,K,rank", [(4, 2, 6, 5, 2), (3, 1, 8, 8, 3), (4, 4, 5, 7, 1), (2, 1, 7, 4, 3)])
def test_decomposition_brute_force(L, G, N, K, rank):
    rng = np.random.default_rng(100 * L + 10 * N + K)
    Ws = [rng.standard_normal((N, K)) for _ in range(L)]
    res = decompose.decompose_family(Ws, num_bands=G, rank=rank, store=False)
    errs, uvs = _brute_decompose([W.tolist() for W in Ws], G, rank)
    assert abs(np.mean(errs) - decompose.mean_error([res])) <= 1e-10
    for l in range(L):
        assert abs(errs[l] - res["err"][l]) <= 1e-10
        uv_b, gap = uvs[l]
        if gap:
            assert np.max(np.abs(uv_b - res["U"][l] @ res["V"][l].T)) <= 1e-9
    # the least-squares scale is a minimum of the row error
    for l in range(L):
        b = decompose.band_of(l, L, G)
        W0 = res["W0"][b]
        for i in range(N):
            f = lambda c: np.sum((Ws[l][i] - c * W0[i]) ** 2)
            sv = res["s"][l][i]
            assert f(sv) <= f(sv + 1e-6) and f(sv) <= f(sv - 1e-6)


def test_zero_shared_row_gets_unit_scale():
    W0 = np.zeros((2, 3))
    W0[1] = [1.0, 2.0, 2.0]
    s = decompose.row_scale(np.array([[1.0, 1.0, 1.0], [2.0, 4.0, 4.0]]), W0)
    assert s[0] == 1.0 and s[1] == 2.0


def test_sanity_band_for_unclustered_layers():
    """P9 (a sanity band, not a pin): two independent N(0, 1/K) layers per band
    give a pre-delta error near sqrt(1/2); a small delta lowers it a little.
    With 26 layers in one band the error is near sqrt(25/26)."""
    rng = np.random.default_rng(5)
    N, K = 256, 128
    Ws = [rng.standard_normal((N, K)) / math.sqrt(K) for _ in range(2)]
    res0 = decompose.decompose_family(Ws, 1, 0, store=False)
    res = decompose.decompose_family(Ws, 1, 8, store=False)
    assert abs(np.mean(res0["err"]) - math.sqrt(0.5)) < 0.03
    assert 0.55 < np.mean(res["err"]) < np.mean(res0["err"])
    Ws26 = [rng.standard_normal((64, 32)) / math.sqrt(32) for _ in range(26)]
    e26 = decompose.mean_error([decompose.decompose_family(Ws26, 1, 0, store=False)])
    assert abs(e26 - math.sqrt(25 / 26)) < 0.03


# --------------------------------------------------------------------------
# ALS refinement of a band ("Quality (Gemma 4 31B)" page, "ALS optimization
# barely helps"; the steps are the reading in oracle/decompose.py)
# --------------------------------------------------------------------------
def _band(rng, m, N, K, spread):
    base = rng.standard_normal((N, K))
    return [base * (1.0 + 0.2 * rng.standard_normal((N, 1))) + spread * rng.standard_normal((N, K))
            for _ in range(m)]


def test_als_zero_sweeps_is_one_shot():
    rng = np.random.default_rng(40)
    Ws = _band(rng, 3, 9, 7, 0.5)
    W0a, ma = decompose.decompose_band(Ws, 2)
    W0b, mb = decompose.als_band(Ws, 2, 0)
    assert np.array_equal(W0a, W0b)
    for x, y in zip(ma, mb):
        for k in ("s", "U", "V"):
            assert np.array_equal(x[k], y[k])


@pytest.mark.parametrize("m,N,K,rank", [(2, 8, 6, 1), (3, 10, 7, 2), (4, 6, 9, 0), (5, 12, 12, 3)])
def test_als_objective_never_increases(m, N, K, rank):
    # block-coordinate descent with exact block minimizers (unrounded)
    rng = np.random.default_rng(41 + m)
    Ws = _band(rng, m, N, K, 0.7)
    prev = None
    for sweeps in range(6):
        W0, mem = decompose.als_band(Ws, rank, sweeps, store=False)
        J = decompose.band_objective(Ws, W0, mem)
        if prev is not None:
            assert J <= prev * (1 + 1e-12) + 1e-12
        prev = J
    # and ALS is not a no-op on a band whose layers differ
    W0, mem = decompose.als_band(Ws, rank, 0, store=False)
    assert prev < decompose.band_objective(Ws, W0, mem) * (1 - 1e-6)


def test_als_shared_block_is_least_squares():
    # the W0 step against a generic least-squares solve of the vectorized
    # problem: unknowns W0[i, j], one equation s_l[i] W0[i, j] = (W_l - D_l)[i, j]
    # per layer and element, built by explicit loops
    rng = np.random.default_rng(43)
    m, N, K = 3, 4, 3
    Ws = [rng.standard_normal((N, K)) for _ in range(m)]
    Ds = [rng.standard_normal((N, K)) * 0.3 for _ in range(m)]
    ss = [rng.standard_normal(N) for _ in range(m)]
    ss[0][2] = ss[1][2] = ss[2][2] = 0.0     # row 2: every scale zero -> keeps the previous row
    prev = rng.standard_normal((N, K))
    got = decompose.shared_block_given(Ws, ss, Ds, prev)
    rows, rhs = [], []
    for l in range(m):
        for i in range(N):
            for j in range(K):
                row = np.zeros(N * K)
                row[i * K + j] = ss[l][i]
                rows.append(row)
                rhs.append(Ws[l][i, j] - Ds[l][i, j])
    sol = np.linalg.lstsq(np.array(rows), np.array(rhs), rcond=None)[0].reshape(N, K)
    live = [0, 1, 3]
    assert np.allclose(got[live], sol[live], rtol=1e-12, atol=1e-12)
    assert np.array_equal(got[2], prev[2])


def test_als_scale_step_is_stationary():
    # after one sweep the scales are the minimizers of J for the W0 and U V^T
    # they were fitted with: a central difference of J in any s_l[i] is zero
    # (the SVD step refits U V^T afterwards, so the check is on J with the
    # sweep's deltas held fixed)
    rng = np.random.default_rng(44)
    Ws = _band(rng, 3, 7, 6, 0.6)
    W0, mem0 = decompose.als_band(Ws, 2, 1, store=False)
    _, mem_prev = decompose.als_band(Ws, 2, 0, store=False)
    Ds = [decompose.delta_product(m["U"], m["V"]) for m in mem_prev]
    for l, (W, D) in enumerate(zip(Ws, Ds)):
        s = mem0[l]["s"]

        def J(sv):
            return float(np.sum((W - sv[:, None] * W0 - D) ** 2))

        for i in range(len(s)):
            h = 1e-5
            e = np.zeros_like(s)
            e[i] = h
            grad = (J(s + e) - J(s - e)) / (2 * h)
            assert abs(grad) < 1e-6 * (1 + J(s))


def test_als_single_layer_band_stays_exact():
    # one layer per band: the one-shot decomposition is exact (W0 = W, s = 1,
    # zero delta) and every sweep keeps it so
    rng = np.random.default_rng(45)
    W = rng.standard_normal((8, 5))
    W0, mem = decompose.als_band([W], 2, 3, store=False)
    assert np.allclose(W0, W, rtol=0, atol=1e-12)
    assert np.allclose(mem[0]["s"], 1.0, rtol=0, atol=1e-12)
    assert mem[0]["err"] < 1e-12


def test_stored_decomposition_dtypes():
    rng = np.random.default_rng(6)
    Ws = [bf16_values(rng, (16, 24)) for _ in range(4)]
    res = decompose.decompose_family(Ws, 2, 3, store=True)
    for b, W0 in res["W0"].items():
        assert np.array_equal(bf16.round_bf16(W0), W0)
    for l in range(4):
        assert np.array_equal(res["s"][l].astype(np.float32).astype(np.float64), res["s"][l])
        assert np.array_equal(bf16.round_bf16(res["U"][l]), res["U"][l])
        assert np.array_equal(bf16.round_bf16(res["V"][l]), res["V"][l])


# --------------------------------------------------------------------------
# bundle sizes printed on the pages
# --------------------------------------------------------------------------
def _gold():
    with open(os.path.join(GOLDEN, "bundle_sizes.json")) as f:
        return json.load(f)


def test_bundle_sizes_match_pages():
    g = _gold()
    shapes = [tuple(v) for v in g["dims"].values()]
    L = g["num_layers"]
    for c in g["checks"]:
        if "value" in c:
            mb = sizes.bundle_mb(shapes, 4, L, 1)["dense"]
            assert abs(mb - c["value"]) <= c["tol"], c["cite"]
        elif "percent" in c:
            m = sizes.bundle_mb(shapes, c["rank"], L, c["G"])
            assert abs(100 * m["theta"] / m["dense"] - c["percent"]) <= c["tol_pct"], c["cite"]
        elif "above" in c:
            m = sizes.bundle_mb(shapes, c["rank"], L, c["G"])
            assert 100 * m["theta"] / m["dense"] > c["above"], c["cite"]
        elif "share_min" in c:
            m = sizes.bundle_mb(shapes, c["rank"], L, c["G"])
            share = 100 * m["W0"] / m["theta"]
            assert c["share_min"] <= share <= c["share_max"], c["cite"]
        elif "below" in c:
            for r in c["ranks"]:
                m = sizes.bundle_mb(shapes, r, L, c["G"])
                assert 100 * m["theta"] / m["dense"] < c["below"], c["cite"]
        else:
            ms = [sizes.bundle_mb(shapes, r, L, c["G"]) for r in c["ranks"]]
            assert len({round(m["W0"], 6) for m in ms}) == 1 and len({round(m["s"], 6) for m in ms}) == 1
            assert ms[0]["U"] < ms[1]["U"] < ms[2]["U"]


def test_bundle_size_closed_forms():
    """The element counts behind the page's table (derived by hand)."""
    shapes = [tuple(v) for v in _gold()["dims"].values()]
    c = sizes.bundle_counts(shapes, 32, 26, 1)
    assert c["dense"] == 444_727_296
    assert c["W0"] == 17_104_896
    assert c["s"] == 26 * 12_032 and c["U"] == 26 * 12_032 * 32 and c["V"] == 26 * 10_880 * 32
    m = sizes.bundle_mb(shapes, 32, 26, 1)
    assert abs(100 * m["W0"] / m["theta"] - 46.9) < 0.05


# --------------------------------------------------------------------------
# tolerance checker
# --------------------------------------------------------------------------
def test_compare_accepts_and_rejects():
    rng = np.random.default_rng(8)
    y = rng.standard_normal((4, 100))
    assert compare.compare(y, y)["ok"]
    assert compare.compare(y * (1 + 1e-3), y)["ok"]
    assert not compare.compare(y * (1 + 1e-2), y)["ok"]           # row error 1e-2 > 5e-3
    bad = y.copy()
    bad[2, 7] += 0.2 * np.abs(y).max()
    assert not compare.compare(bad, y)["ok"]                      # one large element
    z = y.copy()
    z[1] = 0.0
    assert compare.compare(z, z)["ok"]
    w = z.copy()
    w[1, 3] = 1e-6
    assert not compare.compare(w, z)["ok"]                        # zero row must match exactly
    assert not compare.compare(y[:, :50], y)["ok"]
    nan = y.copy()
    nan[0, 0] = np.nan
    assert not compare.compare(nan, y)["ok"]


# ---------------------------------------------------------------------------
# MLP activation of the fused gate|up epilogue ("Quality (Gemma 4 31B)" page,
# "Activation function fix"; "Add a new model architecture" page, "Route the
# MLP through config.hidden_activation")
# ---------------------------------------------------------------------------
_ACT_X = np.concatenate([np.linspace(-9.0, 9.0, 1801), np.random.default_rng(7).normal(0, 3, 500)])


@pytest.mark.parametrize("name", forward.ACTIVATIONS)
def test_activation_matches_library_routines(name):
    """Against independent library routines in fp64: torch's gelu (tanh
    approximation) and silu, and x * Phi(x) from scipy's normal CDF."""
    import scipy.stats
    import torch
    got = forward.activation(name, _ACT_X)
    xt = torch.from_numpy(_ACT_X)
    if name == "gelu_tanh":
        ref = torch.nn.functional.gelu(xt, approximate="tanh").numpy()
    elif name == "silu":
        ref = torch.nn.functional.silu(xt).numpy()
    else:
        ref = _ACT_X * scipy.stats.norm.cdf(_ACT_X)
    assert np.max(np.abs(got - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref)))


def test_activation_closed_forms():
    """act(0) = 0; act(x) -> x for large x and -> 0 for very negative x;
    silu(x) = x (1 + tanh(x/2)) / 2; the tanh approximation stays within
    5e-4 of the exact gelu but is not identical to it."""
    for name in forward.ACTIVATIONS:
        assert forward.activation(name, 0.0) == 0.0
        assert abs(forward.activation(name, 40.0) - 40.0) < 1e-12
        assert abs(forward.activation(name, -40.0)) < 1e-12
    x = np.linspace(-8, 8, 3201)
    assert np.allclose(forward.activation("silu", x), x * (1 + np.tanh(x / 2)) / 2, rtol=0, atol=1e-14)
    d = np.abs(forward.activation("gelu_tanh", x) - forward.activation("gelu", x))
    assert 1e-5 < d.max() < 5e-4


def test_gate_up_act_brute_force():
    """h[t][j] = act(g_tj) u_tj with g, u summed by explicit loops and the
    gelu-tanh written with math.tanh."""
    rng = np.random.default_rng(11)
    T, N, K, r = 2, 3, 5, 2
    gate = (rng.normal(size=(N, K)), rng.normal(1, 0.1, N), rng.normal(size=(N, r)), rng.normal(size=(K, r)))
    up = (rng.normal(size=(N, K)), rng.normal(1, 0.1, N), rng.normal(size=(N, r)), rng.normal(size=(K, r)))
    x = rng.normal(size=(T, K))
    h = forward.gate_up_act(x, gate, up, "gelu_tanh")
    for t in range(T):
        for j in range(N):
            vals = []
            for W0, s, U, V in (gate, up):
                acc = s[j] * sum(W0[j, k] * x[t, k] for k in range(K))
                for q in range(r):
                    acc += U[j, q] * sum(V[k, q] * x[t, k] for k in range(K))
                vals.append(acc)
            g, u = vals
            gelu = 0.5 * g * (1 + math.tanh(math.sqrt(2 / math.pi) * (g + 0.044715 * g ** 3)))
            assert abs(h[t, j] - gelu * u) <= 1e-12 * (1 + abs(gelu * u))


# ---------------------------------------------------------------------------
# FP8 (E4M3) shared block with per-row power-of-two scales (oracle.quant)
# ---------------------------------------------------------------------------
def test_e4m3_table_matches_torch():
    """Every code's value against torch's float8_e4m3fn decoding."""
    import torch
    from oracle import quant
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = quant.E4M3
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.nanmax(got) == 448.0 and np.nanmin(got[got > 0]) == 2.0 ** -9


def test_e4m3_rounding_matches_torch():
    """Round-to-nearest-even encoding against torch's float32 -> float8
    conversion on random, tie and subnormal values within +-448."""
    import torch
    from oracle import quant
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-448, 448, 4000), rng.normal(0, 0.01, 2000),
                        (quant.E4M3[1:126] + quant.E4M3[2:127]) / 2,          # exact ties
                        -(quant.E4M3[1:126] + quant.E4M3[2:127]) / 2, [0.0, 448.0, -448.0, 2.0 ** -10]])
    v = v.astype(np.float32).astype(np.float64)
    got = quant.encode(v)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch maps -0.0 to code 0x80; the oracle stores zero as +0 (code 0) -- same value
    bad = (got != ref) & ~((quant.E4M3[got] == 0) & (quant.E4M3[ref] == 0))
    assert not np.any(bad), v[bad][:5]


def test_row_scale_rule():
    """q = 2^e is the smallest power of two with absmax / q <= 448."""
    from oracle import quant
    for a in [1.0, 448.0, 449.0, 1.75, 1.7500001, 3.5, 2.0 ** -20, 1e-3, 123.456, 7.0e4]:
        e = quant.row_exponent(a)
        assert a / 2.0 ** e <= 448.0 and a / 2.0 ** (e - 1) > 448.0, (a, e)
    assert quant.row_exponent(0.0) == 0
    assert quant.row_exponent(448.0) == 0 and quant.row_exponent(449.0) == 1 and quant.row_exponent(1.0) == -8


def test_quantized_rows_error_bound():
    """Relative error of every element <= 2^-4 (3 mantissa bits, RNE), or
    absolute <= 2^-10 q in the subnormal range; the row maximum is coded
    within [224, 448] q."""
    from oracle import quant
    rng = np.random.default_rng(5)
    W = rng.normal(0, 0.02, (64, 300))
    W[3] = 0.0
    codes, q = quant.quantize_rows(W)
    Wq = quant.dequantize(codes, q)
    err = np.abs(Wq - W)
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(W), 2.0 ** -10 * q[:, None]))
    assert np.all(Wq[3] == 0) and q[3] == 1.0
    m = np.max(np.abs(W), axis=1)[np.arange(64) != 3] / q[np.arange(64) != 3]
    assert np.all((m >= 224.0) & (m <= 448.0))


# --------------------------------------------------------------------------
# MXFP4 shared block (OCP microscaling: E2M1 elements, E8M0 scale per 32)
# --------------------------------------------------------------------------
def _e2m1_from_bits(code):
    """E2M1 value from its bit fields: sign (bit 3), exponent (bits 2-1,
    bias 1), mantissa (bit 0); exponent 0 is subnormal 0.m * 2^(1 - 1)."""
    s = -1.0 if code & 8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    return s * (m * 0.5 if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1))


def test_e2m1_table_from_bit_fields():
    from oracle import quant
    assert [_e2m1_from_bits(c) for c in range(16)] == list(quant.E2M1)
    assert quant.E2M1.max() == 6.0 and sorted(set(np.abs(quant.E2M1))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e2m1_rounding_brute_force():
    """Nearest representable magnitude, ties to the even mantissa (code bit
    0 clear), magnitudes above 6 clamped, by exhaustive search."""
    from oracle import quant
    rng = np.random.default_rng(11)
    mags = np.array([_e2m1_from_bits(c) for c in range(8)])
    ties = (mags[1:] + mags[:-1]) / 2
    v = np.concatenate([rng.uniform(-8, 8, 3000), ties, -ties, [0.0, -0.0, 6.0, 7.9, -100.0]])
    got = quant.e2m1_encode(v)
    for x, c in zip(v, got):
        a = min(abs(x), 6.0)
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        want = want | (8 if (x < 0 and want != 0) else 0)
        assert c == want, (x, c, want)


def test_e8m0_scale_bytes_match_torch():
    """A stored scale byte b stands for 2^(b - 127), as torch decodes E8M0."""
    import torch
    b = np.arange(0, 255, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(ref, 2.0 ** (b.astype(np.int64) - 127))


def test_mx_block_exponent_rule():
    """The shared exponent puts the block maximum in [4, 8) times the scale
    (brute-force search over exponents); all-zero blocks take scale 1."""
    from oracle import quant
    for a in [1.0, 4.0, 7.999, 8.0, 0.013, 2.0 ** -30, 3.0e5, 6.0, 5.99]:
        e = quant.mx_exponent(a)
        brute = [k for k in range(-200, 200) if 4.0 <= a / 2.0 ** k < 8.0]
        assert brute == [e], (a, e, brute)
    codes, scales = quant.quantize_mxfp4(np.zeros((2, 40)))
    assert np.all(codes == 0) and np.all(scales == 127) and codes.shape == (2, 64) and scales.shape == (2, 2)


def test_mxfp4_error_bound():
    """Every element within one scale unit X of its value (the widest E2M1
    gap, 4 to 6, halved) where |w/X| <= 6, within X/4 where |w/X| < 2; the
    block maximum may reach 8X and then saturates to 6X (error < 2X); values
    the format holds are exact; padding columns are zero codes."""
    from oracle import quant
    rng = np.random.default_rng(12)
    W = rng.normal(0, 0.02, (16, 100))
    W[5] = 0.0
    W[6, :32] = 2.0 ** -7 * np.array([_e2m1_from_bits(c % 16) for c in range(32)])   # representable block
    codes, scales = quant.quantize_mxfp4(W)
    D = quant.dequantize_mxfp4(codes, scales, 100)
    X = np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=1)[:, :100]
    err = np.abs(D - W)
    r = np.abs(W) / X
    assert np.all(err[r <= 6] <= X[r <= 6])
    assert np.all((np.abs(D[r > 6]) == 6 * X[r > 6]) & (err[r > 6] < 2 * X[r > 6]))
    small = r < 2.0
    assert np.all(err[small] <= X[small] / 4)
    assert np.array_equal(D[6, :32], W[6, :32]) and np.all(D[5] == 0)
    assert np.all(codes[:, 100:] == 0)
