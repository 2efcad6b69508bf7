"""Pins of the oracle's routing backward (combine_backward, permute_backward,
route_backward): adjoint identities of the linear steps, finite differences
of the forward oracle's own probabilities, closed forms."""
import numpy as np
import pytest

from oracle import moe_oracle as O


def _routing(T, E, K, seed, mask_every=0):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    mask = None
    if mask_every:
        mask = (np.arange(T) % mask_every == 1).astype(np.uint8)
    ids, probs = O.route_topk(logits, K, "softmax", mask=mask)
    perm = O.count_and_permute(ids, 0, E)
    return rng, logits, ids, probs, perm


def test_combine_backward_is_the_adjoint():
    """sum_t <combine(y, p)[t], dout[t]> = sum_r <y[r], d_y[r]> (linear in y),
    and the same form is linear in p with gradient d_probs (exact differences)."""
    T, E, K, H = 50, 8, 3, 16
    rng, _, ids, probs, perm = _routing(T, E, K, 1, mask_every=9)
    s2r = perm["slot_to_row"]
    N = int(perm["offsets"][-1])
    y = rng.standard_normal((N, H))
    dout = rng.standard_normal((T, H))
    p = probs.astype(np.float64)
    dy, dp = O.combine_backward(dout, y, s2r, p, "f64")
    f = lambda pp: float((O.combine(y, s2r, pp, "f64") * dout).sum())
    np.testing.assert_allclose(f(p), float((y * dy).sum()), rtol=1e-12)
    for t, k in [(0, 0), (3, 2), (T - 1, 1), (1, 0)]:
        e = np.zeros_like(p)
        e[t, k] = 1.0
        want = f(p + e) - f(p)   # exact up to rounding: f is linear in p
        np.testing.assert_allclose(dp[t, k], want, rtol=1e-5, atol=1e-6)
    assert (dp[s2r < 0] == 0).all()


def test_combine_backward_brute_force():
    T, E, K, H = 12, 4, 2, 5
    rng, _, ids, probs, perm = _routing(T, E, K, 2)
    s2r = perm["slot_to_row"]
    N = int(perm["offsets"][-1])
    y = rng.standard_normal((N, H))
    dout = rng.standard_normal((T, H))
    dy, dp = O.combine_backward(dout, y, s2r, probs, "f64")
    for t in range(T):
        for k in range(K):
            r = s2r[t, k]
            np.testing.assert_allclose(dy[r], float(probs[t, k]) * dout[t], rtol=1e-15)
            np.testing.assert_allclose(dp[t, k], sum(dout[t, h] * y[r, h] for h in range(H)), rtol=1e-6)


def test_permute_backward_is_the_adjoint():
    """<x_perm(x), g> = <x, permute_backward(g)>."""
    T, E, K, H = 40, 6, 2, 8
    rng, _, ids, probs, perm = _routing(T, E, K, 3, mask_every=7)
    x = rng.standard_normal((T, H))
    xp = O.count_and_permute(ids, 0, E, x)["x_perm"]
    g = rng.standard_normal(xp.shape)
    dx = O.permute_backward(g, perm["slot_to_row"], "f64")
    np.testing.assert_allclose(float((xp * g).sum()), float((x * dx).sum()), rtol=1e-12)
    masked = (np.arange(T) % 7 == 1)
    assert (dx[masked] == 0).all()


def _fd(fn, z, eps=1e-6):
    out = np.zeros_like(z)
    for i in np.ndindex(z.shape):
        zp, zm = z.copy(), z.copy()
        zp[i] += eps
        zm[i] -= eps
        out[i] = (fn(zp) - fn(zm)) / (2 * eps)
    return out


@pytest.mark.parametrize("K", [1, 2, 4])
def test_route_backward_softmax_matches_finite_differences(K):
    rng = np.random.default_rng(10 + K)
    T, E = 6, 8
    logits = rng.standard_normal((T, E))
    ids, probs = O.route_topk(logits.astype(np.float32), K)
    g = rng.standard_normal((T, K))
    dz = O.route_backward(ids, g, "softmax", probs=probs)
    for t in range(T):
        zs = logits[t, ids[t].astype(int)]
        # the float64 softmax of the selected keys (the forward stores fp32)
        fn = lambda zz: float((g[t] * np.exp(zz - zz.max()) / np.exp(zz - zz.max()).sum()).sum())
        np.testing.assert_allclose(dz[t], _fd(fn, zs.astype(np.float64)), rtol=2e-5, atol=1e-6)
        assert abs(float(dz[t].sum())) < 1e-6   # shift invariance of softmax
    if K == 1:
        assert (dz == 0).all()


@pytest.mark.parametrize("scale,with_bias", [(1.0, True), (2.5, False)])
def test_route_backward_sigmoid_matches_finite_differences(scale, with_bias):
    rng = np.random.default_rng(20)
    T, E, K = 5, 12, 4
    logits = rng.standard_normal((T, E))
    b = (rng.standard_normal(E) * 0.3).astype(np.float32) if with_bias else None
    ids, _ = O.route_topk(logits.astype(np.float32), K, "sigmoid", bias=b)
    g = rng.standard_normal((T, K))
    dz = O.route_backward(ids, g, "sigmoid", logits=logits.astype(np.float32), score_bias=b, scale=scale)
    for t in range(T):
        sel = ids[t].astype(int)
        bb = np.zeros(K) if b is None else b[sel].astype(np.float64)

        def fn(zz):
            s = 1.0 / (1.0 + np.exp(-(zz + bb)))
            return float((g[t] * scale * s / s.sum()).sum())
        np.testing.assert_allclose(dz[t], _fd(fn, logits[t, sel].astype(np.float64)), rtol=2e-5, atol=1e-6)


def test_route_backward_grouped_matches_finite_differences_of_the_forward():
    """The group-limited route's gates, taken from the forward oracle itself
    (selection fixed: a step of 1e-4 moves no choice on these logits)."""
    rng = np.random.default_rng(30)
    T, E, K, ng, tg = 4, 32, 4, 4, 2
    logits = rng.standard_normal((T, E)) * 2
    b = (rng.standard_normal(E) * 0.2).astype(np.float32)
    ids, p = O.route_grouped(logits.astype(np.float32), K, ng, tg, bias=b, scale=2.5)
    g = rng.standard_normal((T, K))
    dz = O.route_backward(ids, g, "sigmoid", logits=logits.astype(np.float32), score_bias=None, scale=2.5)
    eps = 1e-4
    for t in range(T):
        sel = ids[t].astype(int)
        for k in range(K):
            zp, zm = logits[t:t + 1].copy(), logits[t:t + 1].copy()
            zp[0, sel[k]] += eps
            zm[0, sel[k]] -= eps
            sp = 1.0 / (1.0 + np.exp(-zp))
            sm = 1.0 / (1.0 + np.exp(-zm))
            ip, pp = O.route_grouped(zp.astype(np.float32), K, ng, tg, bias=b, scale=2.5, scores=sp)
            im, pm = O.route_grouped(zm.astype(np.float32), K, ng, tg, bias=b, scale=2.5, scores=sm)
            assert (ip == ids[t]).all() and (im == ids[t]).all()
            # float64 gates of the fixed selection, recomputed from the float64 scores
            fp = float((g[t] * 2.5 * sp[0, sel] / sp[0, sel].sum()).sum())
            fm = float((g[t] * 2.5 * sm[0, sel] / sm[0, sel].sum()).sum())
            np.testing.assert_allclose(dz[t, k], (fp - fm) / (2 * eps), rtol=1e-4, atol=1e-6)


def test_route_backward_masked_and_invalid_slots():
    ids = np.array([[-1, -1], [3, 1]], np.int16)
    probs = np.array([[0, 0], [0.75, 0.25]], np.float32)
    g = np.array([[5.0, 7.0], [1.0, -1.0]])
    dz = O.route_backward(ids, g, "softmax", probs=probs)
    assert (dz[0] == 0).all()
    # closed form for K = 2: d_z0 = p0 p1 (g0 - g1) = -d_z1
    np.testing.assert_allclose(dz[1], [0.75 * 0.25 * 2.0, -0.75 * 0.25 * 2.0], rtol=1e-6)


def test_mlp_backward_data_matches_torch_autograd():
    """One expert, float64: the data gradient equals torch's autograd of the
    dense SwiGLU MLP (a library routine, independent of the oracle's formulas)."""
    import torch
    rng = np.random.default_rng(40)
    m, H, F = 7, 12, 10
    x = rng.standard_normal((m, H))
    W1 = rng.standard_normal((H, 2 * F)) * 0.3
    W2 = rng.standard_normal((F, H)) * 0.3
    dy = rng.standard_normal((m, H))
    got = O.grouped_mlp_backward_data(x, np.array([0, m]), [W1], [W2], dy, "f64")
    xt = torch.tensor(x, requires_grad=True)
    h = xt @ torch.tensor(W1)
    y = (torch.nn.functional.silu(h[:, :F]) * h[:, F:]) @ torch.tensor(W2)
    y.backward(torch.tensor(dy))
    np.testing.assert_allclose(got, xt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_mlp_backward_data_directional_derivative_and_groups():
    """Several experts with an empty one: <d_x, v> equals the central
    difference of <y(x), d_y> along v (the forward oracle in float64)."""
    rng = np.random.default_rng(41)
    H, F = 8, 6
    counts = [3, 0, 5, 1]
    off = np.concatenate([[0], np.cumsum(counts)])
    N = int(off[-1])
    W1 = [rng.standard_normal((H, 2 * F)) * 0.4 for _ in counts]
    W2 = [rng.standard_normal((F, H)) * 0.4 for _ in counts]
    x = rng.standard_normal((N, H))
    dy = rng.standard_normal((N, H))
    v = rng.standard_normal((N, H))
    dx = O.grouped_mlp_backward_data(x, off, W1, W2, dy, "f64")
    f = lambda xx: float((O.grouped_mlp(xx, off, W1, W2, "f64")[0] * dy).sum())
    eps = 1e-6
    np.testing.assert_allclose(float((dx * v).sum()), (f(x + eps * v) - f(x - eps * v)) / (2 * eps), rtol=1e-6)


def test_swiglu_backward_closed_form():
    """At g = 0: silu'(0) = 1/2 and silu(0) = 0, so d_g = d_a * u / 2, d_u = 0."""
    h = np.array([[0.0, 0.0, 3.0, -2.0]])
    d = O.swiglu_backward(h, np.array([[1.0, 4.0]]), 2)
    np.testing.assert_allclose(d, [[1.5, -4.0, 0.0, 0.0]])


def test_mlp_backward_weights_matches_torch_autograd():
    """Two experts and an empty one, float64: the weight gradients equal
    torch's autograd of each expert's dense SwiGLU MLP; the empty expert's
    are zero."""
    import torch
    rng = np.random.default_rng(42)
    H, F = 10, 6
    counts = [4, 0, 7]
    off = np.concatenate([[0], np.cumsum(counts)])
    W1 = [rng.standard_normal((H, 2 * F)) * 0.3 for _ in counts]
    W2 = [rng.standard_normal((F, H)) * 0.3 for _ in counts]
    x = rng.standard_normal((off[-1], H))
    dy = rng.standard_normal((off[-1], H))
    dW1, dW2 = O.grouped_mlp_backward_weights(x, off, W1, W2, dy, "f64")
    assert (dW1[1] == 0).all() and (dW2[1] == 0).all()
    for e in (0, 2):
        lo, hi = off[e], off[e + 1]
        w1 = torch.tensor(W1[e], requires_grad=True)
        w2 = torch.tensor(W2[e], requires_grad=True)
        h = torch.tensor(x[lo:hi]) @ w1
        y = (torch.nn.functional.silu(h[:, :F]) * h[:, F:]) @ w2
        y.backward(torch.tensor(dy[lo:hi]))
        np.testing.assert_allclose(dW1[e], w1.grad.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dW2[e], w2.grad.numpy(), rtol=1e-12, atol=1e-12)


def _column_grid(rng, m, C, emin=-30, emax=30):
    """[m][C] values on the column-block grid of the MX quantizer: in every
    32-row block of every column, k * 2^e with integers |k| <= 14 and one e per
    (block, column) drawn from [emin, emax].  With the block maximum
    kmax * 2^e the scale exponent is e + floor(log2 kmax) - 8, so every
    element becomes k * 2^(8 - floor(log2 kmax)) <= 448, k with at most 4
    significant bits: an exact E4M3 value.  Exponents differ between the
    columns of a row, so blocks cut along rows are not exact."""
    k = rng.integers(-14, 15, size=(m, C)).astype(np.float64)
    e = rng.integers(emin, emax + 1, size=((m + 31) // 32, C))
    return k * np.ldexp(1.0, np.repeat(e, 32, axis=0)[:m])


def test_weight_gradient_mxfp8_exact_on_column_grid():
    """Operands already on their column-block grid pass the MX quantization
    unchanged, so the MXFP8 weight gradient equals the plain contraction
    X^T d_h, a^T dY (fp32) exactly.  Row-wise blocks (the wrong axis) change
    the same operands."""
    rng = np.random.default_rng(46)
    for m in (1, 31, 32, 70, 128):
        X, a, d_h, dY = (_column_grid(rng, m, C) for C in (64, 32, 64, 64))
        for V in (X, a, d_h, dY):
            np.testing.assert_array_equal(O.weight_gradient_quantize(V), V)
        g1, g2 = O.weight_gradient_contract(X, a, d_h, dY, "mxfp8")
        np.testing.assert_array_equal(g1, (X.T @ d_h).astype(np.float32).astype(np.float64))
        np.testing.assert_array_equal(g2, (a.T @ dY).astype(np.float32).astype(np.float64))
        if m >= 32:
            assert (O.mx_dequantize_rows(*O.mx_quantize_rows(X)) != X).any()


def _spiky_block_column(rng, m, C):
    """[m][C] values whose every 32-row column block is 2^e at its first row and
    s * 2^(e-17) with s in {1, 1.25, 1.5, 1.75} below it, e per column.  The
    block scale is 2^(e-8), so a small value becomes s * 2^-9, an E4M3
    subnormal that rounds to m_s * 2^-9 with m_s = round-half-even(s) = 1,
    1, 2, 2.  Returns (values, their quantized values from that rule)."""
    e = rng.integers(-10, 11, size=C)
    s_choice = rng.integers(0, 4, size=(m, C))
    s = np.array([1.0, 1.25, 1.5, 1.75])[s_choice]
    q = np.array([1.0, 1.0, 2.0, 2.0])[s_choice]
    V = s * np.ldexp(1.0, e - 17)[None, :]
    Q = q * np.ldexp(1.0, e - 17)[None, :]
    first = (np.arange(m) % 32) == 0
    V[first] = np.ldexp(1.0, e)[None, :].repeat(first.sum(), axis=0)
    Q[first] = V[first]
    return V, Q


def _first_rows_zero(V, m):
    V = V.copy()
    V[(np.arange(m) % 32) == 0] = 0.0
    return V


def test_weight_gradient_mxfp8_closed_form_and_planted_mistakes():
    """One operand at a time off the grid, with a closed-form quantization (see
    _spiky_block_column), the others on the grid and zero on the rows that
    hold the blocks' large values, so the gradient comes from the small,
    coarsely quantized values alone.  The oracle equals the closed form
    exactly.  Planted mistakes in the oracle (that operand left unquantized;
    blocks cut along rows instead of columns) move the result by more than
    the 3e-2 MXFP8 tolerance of the GPU tests."""
    rng = np.random.default_rng(47)
    m, H, F = 96, 64, 32
    names = ("X", "a", "d_h", "dY")
    width = {"X": H, "a": F, "d_h": 2 * F, "dY": H}

    def rel(got, want):
        return np.abs(got - want).max() / np.abs(want).max()

    for which in names:
        ops, exact = {}, {}
        for n in names:
            if n == which:
                ops[n], exact[n] = _spiky_block_column(rng, m, width[n])
            else:
                ops[n] = _first_rows_zero(_column_grid(rng, m, width[n], -3, 3), m)
                exact[n] = ops[n]
        g1, g2 = O.weight_gradient_contract(ops["X"], ops["a"], ops["d_h"], ops["dY"], "mxfp8")
        w1 = (exact["X"].T @ exact["d_h"]).astype(np.float32).astype(np.float64)
        w2 = (exact["a"].T @ exact["dY"]).astype(np.float32).astype(np.float64)
        np.testing.assert_array_equal(g1, w1)
        np.testing.assert_array_equal(g2, w2)
        got = g1 if which in ("X", "d_h") else g2
        # mistake 1: the operand is not quantized
        raw = dict(exact)
        raw[which] = ops[which]
        b = raw["X"].T @ raw["d_h"] if which in ("X", "d_h") else raw["a"].T @ raw["dY"]
        assert rel(b, got) > 3e-2, (which, rel(b, got))
        # mistake 2: its blocks run along rows (32 consecutive columns of a row)
        rows = dict(exact)
        rows[which] = O.mx_dequantize_rows(*O.mx_quantize_rows(ops[which]))
        b = rows["X"].T @ rows["d_h"] if which in ("X", "d_h") else rows["a"].T @ rows["dY"]
        assert rel(b, got) > 3e-2, (which, rel(b, got))


def test_weight_gradient_operands_follow_the_data_pass():
    """The weight gradient's a and d_h come from the data pass it follows: for
    a bf16 pass they are the data gradient's bf16 intermediates; for an MXFP8
    pass, those of the MX contractions (the same d_h the MXFP8 data gradient
    feeds into d_x, pinned by its closed form), and the two differ."""
    rng = np.random.default_rng(48)
    H, F, m = 64, 32, 40
    W1 = O.bf16_round(rng.standard_normal((H, 2 * F)) * 0.2)
    W2 = O.bf16_round(rng.standard_normal((F, H)) * 0.2)
    X = O.bf16_round(rng.standard_normal((m, H)))
    dY = O.bf16_round(rng.standard_normal((m, H)))
    for dt in ("bf16", "mxfp8"):
        h, d_a, d_h = O.mlp_backward_intermediates(X, dY, W1, W2, dt)
        Xo, a, dho, dYo = O.weight_gradient_operands(X, dY, W1, W2, dt)
        np.testing.assert_array_equal(Xo, X)
        np.testing.assert_array_equal(dYo, dY)
        np.testing.assert_array_equal(dho, d_h)
        np.testing.assert_array_equal(a, O.bf16_round(O.swiglu(h, F)))
        np.testing.assert_array_equal(d_h, O.bf16_round(O.swiglu_backward(h, d_a, F)))
    hb = O.mlp_backward_intermediates(X, dY, W1, W2, "bf16")[0]
    hm = O.mlp_backward_intermediates(X, dY, W1, W2, "mxfp8")[0]
    assert (hb != hm).any()
    # the full function composes the two steps per expert, empty experts zero
    off = np.array([0, m, m])
    g1, g2 = O.grouped_mlp_backward_weights(X, off, [W1, W1], [W2, W2], dY, "mxfp8", data_dtype="mxfp8")
    c1, c2 = O.weight_gradient_contract(*O.weight_gradient_operands(X, dY, W1, W2, "mxfp8"), "mxfp8")
    np.testing.assert_array_equal(g1[0], c1)
    np.testing.assert_array_equal(g2[0], c2)
    assert (g1[1] == 0).all() and (g2[1] == 0).all()


def test_mlp_backward_weights_mxfp8_within_mx_rounding_of_bf16():
    """General operands: the MXFP8 weight gradient stays within the E4M3
    rounding of the bf16 one (four quantized operands, RMS relative error
    about 2^-4 / sqrt(3) each: about 0.07 in all; bound 0.1)."""
    rng = np.random.default_rng(43)
    H, F = 64, 32
    counts = [40, 0, 33]
    off = np.concatenate([[0], np.cumsum(counts)])
    W1 = [O.bf16_round(rng.standard_normal((H, 2 * F)) * 0.1) for _ in counts]
    W2 = [O.bf16_round(rng.standard_normal((F, H)) * 0.1) for _ in counts]
    x = O.bf16_round(rng.standard_normal((off[-1], H)))
    dy = O.bf16_round(rng.standard_normal((off[-1], H)))
    b1, b2 = O.grouped_mlp_backward_weights(x, off, W1, W2, dy, "bf16")
    m1, m2 = O.grouped_mlp_backward_weights(x, off, W1, W2, dy, "mxfp8")
    assert np.linalg.norm(m1 - b1) <= 0.1 * np.linalg.norm(b1) and np.linalg.norm(m2 - b2) <= 0.1 * np.linalg.norm(b2)
    assert (m1[1] == 0).all() and (m2[1] == 0).all()


def test_mlp_backward_data_mxfp8_large_gate_closed_form():
    """The MXFP8 data gradient on operands that every MX quantization keeps
    exactly: one-hot rows of x (+1) and d_y (+-1), W1's gate columns all 16,
    its up columns and W2 in {-2..2}.  Then g = 16 and u, d_a are small
    integers; silu(16) and silu'(16) equal 16 and 1 to within 2e-6, below half
    a bf16 step of the stored d_h, so d_h = [d_a u, 16 d_a] exactly and
    d_x = bf16(d_a u . W1_gate^T + 16 d_a . W1_up^T) in integers; the bf16
    path gives the same."""
    rng = np.random.default_rng(44)
    H, F = 64, 32
    counts = [5, 0, 9]
    off = np.concatenate([[0], np.cumsum(counts)])
    N = int(off[-1])
    W1 = [np.concatenate([np.full((H, F), 16.0), rng.integers(-2, 3, (H, F)).astype(np.float64)], axis=1)
          for _ in counts]
    W2 = [rng.integers(-2, 3, (F, H)).astype(np.float64) for _ in counts]
    x = np.zeros((N, H))
    x[np.arange(N), rng.integers(0, H, N)] = 1.0
    dy = np.zeros((N, H))
    dy[np.arange(N), rng.integers(0, H, N)] = rng.choice([-1.0, 1.0], N)
    got = O.grouped_mlp_backward_data(x, off, W1, W2, dy, "mxfp8")
    want = np.zeros((N, H))
    for e in range(len(counts)):
        lo, hi = off[e], off[e + 1]
        u = x[lo:hi] @ W1[e][:, F:]
        d_a = dy[lo:hi] @ W2[e].T
        want[lo:hi] = O.bf16_round((d_a * u) @ W1[e][:, :F].T + (16.0 * d_a) @ W1[e][:, F:].T)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(O.grouped_mlp_backward_data(x, off, W1, W2, dy, "bf16"), want)


def test_mlp_backward_data_mxfp8_within_mx_rounding_of_f64():
    """General operands: the MXFP8 data gradient stays within the E4M3
    rounding of the float64 chain rule (six quantized operands, each with an
    RMS relative error of about 2^-4 / sqrt(3): about sqrt(6) * 0.036 = 0.09
    in all; bound 0.12), and a transposed W2 (a plausible mistake) does not."""
    rng = np.random.default_rng(45)
    H, F = 64, 64
    counts = [37, 0, 64]
    off = np.concatenate([[0], np.cumsum(counts)])
    W1 = [O.bf16_round(rng.standard_normal((H, 2 * F)) * 0.2) for _ in counts]
    W2 = [O.bf16_round(rng.standard_normal((F, H)) * 0.2) for _ in counts]
    x = O.bf16_round(rng.standard_normal((off[-1], H)))
    dy = O.bf16_round(rng.standard_normal((off[-1], H)))
    ref = O.grouped_mlp_backward_data(x, off, W1, W2, dy, "f64")
    got = O.grouped_mlp_backward_data(x, off, W1, W2, dy, "mxfp8")
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel <= 0.12
    bad = O.grouped_mlp_backward_data(x, off, W1, [w.T.copy() for w in W2], dy, "f64")
    assert np.linalg.norm(bad - ref) / np.linalg.norm(ref) > 0.5
