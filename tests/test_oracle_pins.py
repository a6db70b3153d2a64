"""Pins of the fp64 CPU oracle against facts fixed outside the oracle itself.

Each pin is chosen so that a plausible slip in the oracle (a dropped scale,
a softmax over the wrong axis, a transposed operand, values instead of Z in
the decode, a missing FLARE++ residual) fails at least one test:

* library routine: the FLARE pages state that both stages are standard
  scaled-dot-product attention calls (FLARE arXiv abstract; FLARE++ arXiv
  abstract), so encode, decode, FLARE and FLARE++ are compared with torch's
  float64 ``scaled_dot_product_attention`` on the CPU;
* closed forms: one token, one latent, zero queries, and two-token sigmoid
  cases worked out by hand below;
* invariants of the token-mixing matrix W = A_dec A_enc, which the FLARE
  abstract says has rank at most M: row-stochastic, non-negative, rank <= M,
  reversible (detailed balance) with real eigenvalues in [0, 1], Y = W V;
* equivariance under token permutations, constant V, and linearity in V
  (FLARE only; FLARE++ is not linear in V).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from flare_inputs import f32_to_bf16_bits, make_inputs

RNG = np.random.default_rng(1234)


def rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def sdpa(q, k, v):
    """torch float64 SDPA with its default scale 1/sqrt(head width)."""
    out = F.scaled_dot_product_attention(torch.from_numpy(np.array(q, dtype=np.float64)),
                                         torch.from_numpy(np.array(k, dtype=np.float64)),
                                         torch.from_numpy(np.array(v, dtype=np.float64)))
    return out.numpy()


# ------------------------------------------------------------ library routine
@pytest.mark.parametrize("B,H,N,M,D", [(2, 3, 37, 5, 8), (1, 2, 130, 17, 16), (1, 1, 1, 1, 4)])
def test_encode_is_sdpa_of_latents_over_tokens(B, H, N, M, D):
    Q, K, V = rand(H, M, D), rand(B, H, N, D), rand(B, H, N, D)
    Z = oracle.encode(Q, K, V)
    ref = sdpa(np.broadcast_to(Q, (B, H, M, D)), K, V)
    np.testing.assert_allclose(Z, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("B,H,N,M,D", [(2, 3, 37, 5, 8), (1, 2, 65, 33, 16)])
def test_decode_is_sdpa_of_tokens_over_latents(B, H, N, M, D):
    Q, K, Z = rand(H, M, D), rand(B, H, N, D), rand(B, H, M, D)
    Y = oracle.decode(Q, K, Z)
    ref = sdpa(K, np.broadcast_to(Q, (B, H, M, D)), Z)
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-13)


def test_forward_is_two_sdpa_calls():
    B, H, N, M, D = 2, 2, 50, 7, 8
    Q, K, V = rand(H, M, D, scale=0.7), rand(B, H, N, D), rand(B, H, N, D)
    Y, Z = oracle.forward(Q, K, V)
    Qb = np.broadcast_to(Q, (B, H, M, D))
    Zr = sdpa(Qb, K, V)
    np.testing.assert_allclose(Z, Zr, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Y, sdpa(K, Qb, Zr), rtol=1e-12, atol=1e-13)


def test_pp_forward_is_residual_then_two_sdpa_calls():
    B, H, N, M, D = 2, 2, 40, 6, 8
    Q, K, V = rand(H, M, D, scale=0.5), rand(B, H, N, D), rand(B, H, N, D)
    Y, Qp, Z = oracle.pp_forward(Q, K, V)
    Qb = np.broadcast_to(Q, (B, H, M, D))
    Qp_ref = Qb + sdpa(Qb, K, V)
    Z_ref = sdpa(Qp_ref, K, V)
    np.testing.assert_allclose(Qp, Qp_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Z, Z_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Y, sdpa(K, Qp_ref, Z_ref), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- closed forms
def test_single_token_encode_returns_that_token():
    Q, K, V = rand(3, 9, 8), rand(1, 3, 1, 8), rand(1, 3, 1, 8)
    Z = oracle.encode(Q, K, V)
    np.testing.assert_array_equal(Z, np.broadcast_to(V, (1, 3, 9, 8)))
    Y, _ = oracle.forward(Q, K, V)
    np.testing.assert_allclose(Y, V, rtol=0, atol=1e-15)


def test_zero_queries_give_token_means():
    B, H, N, M, D = 1, 2, 33, 4, 8
    K, V = rand(B, H, N, D), rand(B, H, N, D)
    Q = np.zeros((H, M, D))
    Y, Z = oracle.forward(Q, K, V)
    mean = V.mean(axis=2, keepdims=True)
    np.testing.assert_allclose(Z, np.broadcast_to(mean, Z.shape), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Y, np.broadcast_to(mean, Y.shape), rtol=1e-13, atol=1e-14)


def test_single_latent_decode_copies_z():
    Q, K, Z = rand(2, 1, 8), rand(1, 2, 21, 8), rand(1, 2, 1, 8)
    Y = oracle.decode(Q, K, Z)
    np.testing.assert_array_equal(Y, np.broadcast_to(Z, Y.shape))


def sigmoid(x):
    return 1.0 / (1.0 + math.exp(-x))


@pytest.mark.parametrize("q", [-2.0, -0.3, 0.0, 0.9, 3.0])
def test_two_token_closed_forms(q):
    # D=4 (s=1/2). Tokens k0 = 0 and k1 = e0; one latent q*e0. The encode is a
    # two-way softmax of logits 0 and q/2, so with values v0 = 0, v1 = e1 it
    # gives Z = sigmoid(q/2) e1 (e1 keeps K and V apart), and with one latent
    # every token decodes to Z. For FLARE++ take v1 = e0: the first encode
    # gives sigmoid(q/2) e0, the corrected latent is q' = q + sigmoid(q/2)
    # along e0, and the result is sigmoid(q'/2) e0 for every token.
    D = 4
    K = np.zeros((1, 1, 2, D)); K[0, 0, 1, 0] = 1.0
    V = np.zeros((1, 1, 2, D)); V[0, 0, 1, 1] = 1.0
    Q = np.zeros((1, 1, D)); Q[0, 0, 0] = q
    Y, Z = oracle.forward(Q, K, V)
    z = sigmoid(q / 2.0)
    exp_z = np.zeros(D); exp_z[1] = z
    np.testing.assert_allclose(Z[0, 0, 0], exp_z, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(Y[0, 0], np.broadcast_to(exp_z, (2, D)), rtol=1e-14, atol=1e-15)

    Vpp = np.zeros((1, 1, 2, D)); Vpp[0, 0, 1, 0] = 1.0
    Ypp, Qp, Zpp = oracle.pp_forward(Q, K, Vpp)
    qp = q + sigmoid(q / 2.0)
    np.testing.assert_allclose(Qp[0, 0, 0, 0], qp, rtol=1e-14)
    np.testing.assert_allclose(Ypp[0, 0, :, 0], [sigmoid(qp / 2.0)] * 2, rtol=1e-14)
    # without the residual the answer would be sigmoid(sigmoid(q/2)/2); the two
    # readings coincide only at q = 0
    if q != 0.0:
        assert abs(sigmoid(qp / 2.0) - sigmoid(sigmoid(q / 2.0) / 2.0)) > 1e-3


@pytest.mark.parametrize("a,b", [(1.0, -1.0), (0.2, 2.5)])
def test_two_latent_decode_closed_form(a, b):
    # D=1 (s=1): token k attends to latents a and b with logits a*k and b*k,
    # so its weight on latent a is sigmoid((a - b) k).
    ks = np.array([-1.5, 0.0, 0.4, 2.0])
    Q = np.array([[[a], [b]]])
    K = ks.reshape(1, 1, 4, 1)
    Z = np.array([[[[3.0], [-1.0]]]])
    Y = oracle.decode(Q, K, Z)
    w = np.array([sigmoid((a - b) * k) for k in ks])
    np.testing.assert_allclose(Y[0, 0, :, 0], w * 3.0 + (1 - w) * -1.0, rtol=1e-14, atol=1e-15)


# -------------------------------------------------------- mixing-matrix facts
def mixing_matrix(Q, K):
    """W (N x N) read off the oracle: Y columns are W applied to V columns."""
    N, D = K.shape
    assert D >= N
    V = np.zeros((N, D))
    V[:, :N] = np.eye(N)
    Z = oracle.encode_head(Q, K, V)
    Y = oracle.decode_head(Q, K, Z)
    return Y[:, :N]


@pytest.mark.parametrize("N,M", [(12, 3), (16, 5), (10, 1)])
def test_mixing_matrix_is_reversible_stochastic_and_low_rank(N, M):
    D = 16
    Q, K = rand(M, D, scale=0.8), rand(N, D)
    W = mixing_matrix(Q, K)
    assert (W >= 0).all()
    np.testing.assert_allclose(W.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    sv = np.linalg.svd(W, compute_uv=False)
    assert sv[M] / sv[0] < 1e-12 if M < N else True
    assert sv[M - 1] / sv[0] > 1e-8  # rank exactly M for generic inputs
    # stationary distribution pi (left eigenvector of eigenvalue 1)
    evals, evecs = np.linalg.eig(W.T)
    i = np.argmin(abs(evals - 1.0))
    pi = np.real(evecs[:, i]); pi = pi / pi.sum()
    assert (pi > 0).all()
    F_ = pi[:, None] * W
    np.testing.assert_allclose(F_, F_.T, rtol=0, atol=1e-14)
    assert np.max(abs(np.imag(evals))) < 1e-10
    ev = np.real(evals)
    assert ev.min() > -1e-10 and ev.max() < 1 + 1e-10
    # Y = W V for an arbitrary V
    V = rand(N, D)
    Y = oracle.decode_head(Q, K, oracle.encode_head(Q, K, V))
    np.testing.assert_allclose(Y, W @ V, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("pp", [False, True])
def test_token_permutation_permutes_output(pp):
    B, H, N, M, D = 1, 2, 45, 6, 8
    Q, K, V = rand(H, M, D, scale=0.6), rand(B, H, N, D), rand(B, H, N, D)
    perm = RNG.permutation(N)
    f = (lambda *a: oracle.pp_forward(*a)[0]) if pp else (lambda *a: oracle.forward(*a)[0])
    Y = f(Q, K, V)
    Yp = f(Q, K[:, :, perm], V[:, :, perm])
    np.testing.assert_allclose(Yp, Y[:, :, perm], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("pp", [False, True])
def test_constant_values_give_constant_output(pp):
    B, H, N, M, D = 2, 2, 30, 5, 8
    Q, K = rand(H, M, D), rand(B, H, N, D)
    c = rand(B, H, 1, D)
    V = np.broadcast_to(c, (B, H, N, D)).copy()
    Y = oracle.pp_forward(Q, K, V)[0] if pp else oracle.forward(Q, K, V)[0]
    np.testing.assert_allclose(Y, np.broadcast_to(c, Y.shape), rtol=1e-13, atol=1e-14)


def test_flare_is_linear_in_values_and_flarepp_is_not():
    B, H, N, M, D = 1, 1, 40, 4, 8
    Q, K = rand(H, M, D), rand(B, H, N, D)
    V1, V2 = rand(B, H, N, D), rand(B, H, N, D)
    a, b = 0.7, -1.3
    Y = lambda V: oracle.forward(Q, K, V)[0]
    np.testing.assert_allclose(Y(a * V1 + b * V2), a * Y(V1) + b * Y(V2), rtol=1e-11, atol=1e-12)
    P = lambda V: oracle.pp_forward(Q, K, V)[0]
    assert np.max(abs(P(a * V1 + b * V2) - (a * P(V1) + b * P(V2)))) > 1e-3


def test_sampled_rows_match_full_decode():
    Q, K, V = rand(2, 5, 8), rand(1, 2, 50, 8), rand(1, 2, 50, 8)
    Y, Z = oracle.forward(Q, K, V)
    rows = np.array([49, 0, 17, 17, 3])
    Ys, _ = oracle.forward(Q, K, V, rows=rows)
    np.testing.assert_array_equal(Ys, Y[:, :, rows])


# ------------------------------------------------------- input widening / gen
def test_bf16_widening_matches_torch():
    x = RNG.standard_normal(4096).astype(np.float32) * 3
    bits = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.widen(bits), ref)


def test_generator_is_deterministic_and_shaped():
    a = make_inputs(2, 3, 100, 7, 16, "bf16", 0.5, 1.0, seed=9)
    b = make_inputs(2, 3, 100, 7, 16, "bf16", 0.5, 1.0, seed=9)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert a[0].shape == (3, 7, 16) and a[1].shape == (2, 3, 100, 16) and a[0].dtype == np.uint16
    q32 = make_inputs(1, 1, 8, 4, 16, "f32", 2.0, 1.0, seed=3)[0]
    assert q32.dtype == np.float32 and 1.0 < q32.std() < 3.0


# ------------------------------------------ token-query decode (skill page)
@pytest.mark.parametrize("B,H,N,M,D", [(2, 3, 37, 5, 8), (1, 2, 65, 33, 16), (1, 1, 1, 1, 4)])
def test_attend_is_sdpa_of_token_queries_over_latent_states(B, H, N, M, D):
    q, Z = rand(B, H, N, D), rand(B, H, M, D)
    np.testing.assert_allclose(oracle.attend(q, Z), sdpa(q, Z, Z), rtol=1e-12, atol=1e-13)


def test_attend_single_latent_and_zero_queries():
    q, Z1 = rand(1, 2, 9, 8), rand(1, 2, 1, 8)
    Y = oracle.attend(q, Z1)
    np.testing.assert_allclose(Y, np.broadcast_to(Z1, Y.shape), rtol=1e-15, atol=0)
    Z = rand(1, 2, 6, 8)
    Y0 = oracle.attend(np.zeros((1, 2, 5, 8)), Z)
    np.testing.assert_allclose(Y0, np.broadcast_to(Z.mean(axis=2, keepdims=True), Y0.shape), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("a,b", [(1.0, -1.0), (0.3, 2.0)])
def test_attend_two_latent_closed_form(a, b):
    # D=1 (s=1): token query x has logits a*x and b*x against latent states a
    # and b, so Y = w*a + (1-w)*b with w = sigmoid((a - b) x).
    xs = np.array([-2.0, -0.1, 0.0, 1.3])
    q = xs.reshape(1, 1, 4, 1)
    Z = np.array([[[[a], [b]]]])
    w = np.array([sigmoid((a - b) * x) for x in xs])
    np.testing.assert_allclose(oracle.attend(q, Z)[0, 0, :, 0], w * a + (1 - w) * b, rtol=1e-14, atol=1e-15)


# ------------------------------------------------------------------ backward
def torch_flare_grads(Q, K, V, dY):
    """Gradients of sum(Y * dY) for Y = FLARE(Q, K, V), by torch fp64 autograd through two SDPA calls
    (Q shared over the batch)."""
    q = torch.tensor(Q, dtype=torch.float64, requires_grad=True)
    k = torch.tensor(K, dtype=torch.float64, requires_grad=True)
    v = torch.tensor(V, dtype=torch.float64, requires_grad=True)
    qb = q.unsqueeze(0).expand(k.shape[0], -1, -1, -1)
    z = F.scaled_dot_product_attention(qb, k, v)
    y = F.scaled_dot_product_attention(k, qb, z)
    (y * torch.tensor(dY, dtype=torch.float64)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("B,H,N,M,D", [(2, 2, 37, 5, 8), (1, 1, 70, 33, 16), (1, 1, 1, 1, 4)])
def test_backward_is_autograd_of_two_sdpa_calls(B, H, N, M, D):
    Q, K, V, dY = rand(H, M, D), rand(B, H, N, D), rand(B, H, N, D), rand(B, H, N, D)
    got = oracle.backward(Q, K, V, dY)
    want = torch_flare_grads(Q, K, V, dY)
    for g, w, name in zip(got, want, ("dQ", "dK", "dV")):
        np.testing.assert_allclose(g, w, rtol=1e-10, atol=1e-12, err_msg=name)


def test_backward_matches_central_differences_of_the_forward():
    B, H, N, M, D = 1, 1, 5, 3, 4
    Q, K, V, dY = rand(H, M, D), rand(B, H, N, D), rand(B, H, N, D), rand(B, H, N, D)
    dQ, dK, dV = oracle.backward(Q, K, V, dY)

    def f(q, k, v):
        return float(np.sum(oracle.forward(q, k, v)[0] * dY))

    h = 1e-6
    for arr, grad in ((Q, dQ), (K, dK), (V, dV)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a0 = arr[idx]
            arr[idx] = a0 + h
            fp = f(Q, K, V)
            arr[idx] = a0 - h
            fm = f(Q, K, V)
            arr[idx] = a0
            fd[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8)


# ------------------------------------------------------------ FLARE++ backward
def torch_pp_grads(Q, K, V, dY):
    """Gradients of sum(Y * dY) for Y = FLARE++(Q, K, V), by torch fp64 autograd through three SDPA
    calls: Z0 = SDPA(Q, K, V), Q' = Q + Z0, Y = SDPA(K, Q', SDPA(Q', K, V)) (Q shared over the batch)."""
    q = torch.tensor(Q, dtype=torch.float64, requires_grad=True)
    k = torch.tensor(K, dtype=torch.float64, requires_grad=True)
    v = torch.tensor(V, dtype=torch.float64, requires_grad=True)
    qb = q.unsqueeze(0).expand(k.shape[0], -1, -1, -1)
    qp = qb + F.scaled_dot_product_attention(qb, k, v)
    z = F.scaled_dot_product_attention(qp, k, v)
    y = F.scaled_dot_product_attention(k, qp, z)
    (y * torch.tensor(dY, dtype=torch.float64)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("N,M,D", [(37, 5, 8), (70, 33, 16), (1, 1, 4)])
def test_encode_backward_is_autograd_of_one_sdpa_call(N, M, D):
    Q, K, V, dZ = rand(M, D), rand(N, D), rand(N, D), rand(M, D)
    got = oracle.encode_backward_head(Q, K, V, dZ)
    q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    (F.scaled_dot_product_attention(q, k, v) * torch.tensor(dZ, dtype=torch.float64)).sum().backward()
    for g, w, name in zip(got, (q.grad.numpy(), k.grad.numpy(), v.grad.numpy()), ("dQ", "dK", "dV")):
        np.testing.assert_allclose(g, w, rtol=1e-10, atol=1e-12, err_msg=name)


@pytest.mark.parametrize("B,H,N,M,D", [(2, 2, 37, 5, 8), (1, 1, 70, 33, 16), (1, 1, 1, 1, 4)])
def test_pp_backward_is_autograd_of_three_sdpa_calls(B, H, N, M, D):
    Q, K, V, dY = rand(H, M, D), rand(B, H, N, D), rand(B, H, N, D), rand(B, H, N, D)
    got = oracle.pp_backward(Q, K, V, dY)
    want = torch_pp_grads(Q, K, V, dY)
    for g, w, name in zip(got, want, ("dQ", "dK", "dV")):
        np.testing.assert_allclose(g, w, rtol=1e-10, atol=1e-12, err_msg=name)


def test_pp_backward_matches_central_differences_of_the_forward():
    B, H, N, M, D = 2, 1, 5, 3, 4
    Q, K, V, dY = rand(H, M, D), rand(B, H, N, D), rand(B, H, N, D), rand(B, H, N, D)
    dQ, dK, dV = oracle.pp_backward(Q, K, V, dY)

    def f(q, k, v):
        return float(np.sum(oracle.pp_forward(q, k, v)[0] * dY))

    h = 1e-6
    for arr, grad in ((Q, dQ), (K, dK), (V, dV)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a0 = arr[idx]
            arr[idx] = a0 + h
            fp = f(Q, K, V)
            arr[idx] = a0 - h
            fm = f(Q, K, V)
            arr[idx] = a0
            fd[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8)


def test_pp_backward_differs_from_the_flare_backward():
    # the first stage contributes: dropping it (the FLARE backward at Q' alone) changes every gradient
    B, H, N, M, D = 1, 1, 20, 4, 8
    Q, K, V, dY = rand(H, M, D), rand(B, H, N, D), rand(B, H, N, D), rand(B, H, N, D)
    pp = oracle.pp_backward(Q, K, V, dY)
    Qp = oracle.pp_forward(Q, K, V)[1][:, :, :, :].reshape(B, H, M, D)[0]
    second = oracle.backward(Qp, K, V, dY)
    for a, b in zip(pp, second):
        assert np.max(np.abs(a - b)) > 1e-3
