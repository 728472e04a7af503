"""The oracle's backward is pinned to its forward: every gradient it returns
matches central finite differences of L = sum(d_out * out) computed through
the oracle forward (fp64 arithmetic on fp32 inputs perturbed by an exactly
representable step), on the tiny workload with random RMSNorm gains, several
branches (shared and separate queries), a populated conv state and the
residual flag.  The gather's adjoint is checked against the gather itself."""
import numpy as np
import pytest

from synth import workloads as W

STEP = 2.0 ** -12


def _setup(nb, nbh, with_state, seed):
    w = W.get("tiny").replace(batch=2, seq_len=20, n_branches=nb)
    ids, hist = W.make_ids(w)
    rs = np.random.default_rng(seed)
    n, d, mem = ids.size, w.hidden, w.mem_dim
    p = dict(
        tables=[W.table_values(w, j).copy() for j in range(w.n_tables)],
        hidden=rs.standard_normal((n, nbh, d)).astype(np.float32),
        wk=(rs.standard_normal((nb, mem, d)) / np.sqrt(mem)).astype(np.float32),
        wv=(rs.standard_normal((mem, d)) / np.sqrt(mem)).astype(np.float32),
        conv_w=(rs.standard_normal((4, d)) * 0.5).astype(np.float32),
        gamma_q=(1 + 0.1 * rs.standard_normal(d)).astype(np.float32),
        gamma_k=(1 + 0.1 * rs.standard_normal(d)).astype(np.float32),
        gamma_u=(1 + 0.1 * rs.standard_normal(d)).astype(np.float32),
    )
    state = (rs.standard_normal((w.batch, 3 * w.max_order, nb, d)) if with_state else None)
    d_out = rs.standard_normal((n, nb, d))
    return w, ids, hist, p, state, d_out


def _loss(orc, w, ids, hist, p, state, d_out, residual):
    f = orc.forward(ids, hist, W.make_lut(w), w.vocab, w.vocab_compressed, w.orders, w.heads,
                    w.rows(), W.hash_multipliers(w), p["tables"], p["hidden"], p["wk"], p["wv"],
                    p["conv_w"], "f32", gamma_q=p["gamma_q"], gamma_k=p["gamma_k"],
                    gamma_u=p["gamma_u"], eps=w.rms_eps, conv_state=state)
    out = f["delta"]
    if residual:
        h = p["hidden"].astype(np.float64)
        out = out + (h if h.shape[1] == out.shape[1] else h[:, :1])
    return float((d_out * out).sum())


def _fd(orc, w, ids, hist, p, state, d_out, residual, name, index):
    arr = p[name][index[0]] if name == "tables" else p[name]
    idx = index[1:] if name == "tables" else index
    x0 = arr[idx]
    vals = []
    for sgn in (1, -1):
        arr[idx] = np.float32(x0 + sgn * STEP)
        assert float(arr[idx]) == float(x0) + sgn * STEP  # the step is exact in fp32
        vals.append(_loss(orc, w, ids, hist, p, state, d_out, residual))
    arr[idx] = x0
    return (vals[0] - vals[1]) / (2 * STEP)


@pytest.mark.parametrize("nb,nbh,with_state,residual", [(1, 1, False, False), (1, 1, True, True),
                                                        (2, 1, False, True), (2, 2, True, False)])
def test_backward_matches_finite_differences(orc, nb, nbh, with_state, residual):
    w, ids, hist, p, state, d_out = _setup(nb, nbh, with_state, seed=nb * 10 + nbh)
    g = orc.backward(ids, hist, W.make_lut(w), w.vocab, w.vocab_compressed, w.orders, w.heads,
                     w.rows(), W.hash_multipliers(w), p["tables"], p["hidden"], p["wk"], p["wv"],
                     p["conv_w"], "f32", d_out, gamma_q=p["gamma_q"], gamma_k=p["gamma_k"],
                     gamma_u=p["gamma_u"], eps=w.rms_eps, conv_state=state, add_residual=residual)
    rs = np.random.default_rng(7)
    checks = []
    # table entries in rows the tokens hit (one row hit by several tokens too)
    for j in range(w.n_tables):
        rows_j, grads_j = g["d_tables"][j]
        counts = np.bincount(g["row_idx"][:, j], minlength=w.rows()[j])[rows_j]
        for k in [int(np.argmax(counts)), int(rs.integers(len(rows_j)))]:
            c = int(rs.integers(w.row_dim))
            checks.append(("tables", (j, int(rows_j[k]), c), grads_j[k, c]))
    for name, grad in [("wk", g["d_wk"]), ("wv", g["d_wv"]), ("conv_w", g["d_conv_w"]),
                       ("hidden", g["d_hidden"]), ("gamma_q", g["d_gamma_q"]),
                       ("gamma_k", g["d_gamma_k"]), ("gamma_u", g["d_gamma_u"])]:
        for _ in range(3):
            idx = tuple(int(rs.integers(s)) for s in grad.shape)
            checks.append((name, idx, grad[idx]))
    scale = max(abs(c[2]) for c in checks)
    for name, idx, analytic in checks:
        fd = _fd(orc, w, ids, hist, p, state, d_out, residual, name, idx)
        assert abs(fd - analytic) <= 1e-6 * scale + 1e-5 * abs(analytic), (name, idx, fd, analytic)


def test_scatter_is_the_gathers_adjoint(orc):
    """<gather(T), dE> = <T, scatter(dE)> for random tables T and dE, with
    rows hit many times (a skewed row distribution)."""
    rs = np.random.default_rng(11)
    nt, rows, row_dim, n = 3, 40, 16, 500
    row_idx = (rs.zipf(1.5, (n, nt)) % rows).astype(np.int32)
    tabs = [rs.standard_normal((rows, row_dim)).astype(np.float32) for _ in range(nt)]
    d_e = rs.standard_normal((n, nt * row_dim))
    lhs = float((orc.gather(row_idx, tabs, "f32") * d_e).sum())
    rhs = 0.0
    for j, (r, gr) in enumerate(orc.scatter_add(row_idx, d_e, row_dim)):
        rhs += float((tabs[j][r].astype(np.float64) * gr).sum())
        # brute force: each row's gradient is the sum of the slices of the tokens naming it
        for k in range(len(r)):
            want = d_e[row_idx[:, j] == r[k], j * row_dim:(j + 1) * row_dim].sum(axis=0)
            assert np.allclose(gr[k], want, rtol=0, atol=1e-12)
    assert abs(lhs - rhs) <= 1e-9 * abs(lhs)
