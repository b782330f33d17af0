"""Pins of the oracle's Decoupled AdamW (DeToNATION notes, "Decoupled AdamW":
first and second moments kept local, not synchronised) against closed forms
and against torch.optim.AdamW (float64) where the method reduces to it.

The reading checked here: m = beta1*m + (1-beta1)*g goes through the usual
extraction and error feedback; v = beta2*v + (1-beta2)*g^2; the exchanged Q
updates theta -= eta*((Q/(1-beta1^t)) / (sqrt(v/(1-beta2^t)) + eps) + wd*theta)
with t = step + 1.  The slots carry values (sign off); the sign-on
configuration is refused.
"""
import numpy as np
import pytest

import oracle
from oracle import DCT, DILOCO, RANDOM, AdamW, Params, Shard

N = 32
F = np.float64


def f32(x):
    return F(np.float32(x))


def _state(L, seed):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(L).astype(np.float32)
    th = (rng.standard_normal(L) * 0.02).astype(np.float32)
    return g, th


@pytest.mark.parametrize("gscale,eps", [(1.0, 1e-8), (1e-3, 1e-3)])
def test_first_step_is_eta_times_normalised_gradient_plus_decay(gscale, eps):
    """t = 1 from zero moments: v_hat = g^2 and Q_hat = g (all 32 slots, values
    sent as fp32), so the step is eta*(g/(|g| + eps) + wd*theta); eps as large
    as |g| makes its place (outside the square root) visible."""
    L = 32 * 20
    g, th = _state(L, 1)
    g = (g * np.float32(gscale)).astype(np.float32)
    w = AdamW(beta2=0.999, eps=eps, weight_decay=0.01)
    p = Params(scheme=RANDOM, k=32, sign=0, value_fmt=oracle.F32, beta=0.9, lr=1e-3, step=0)
    sh = Shard.contiguous(L, np.zeros(L, np.float32), th)
    idx, val, q, _ = sh.encode(p, oracle.pad_chunks(g, L), w)
    sh.decode(p, [idx], [val], w)
    gg = g.astype(F).reshape(-1, N)
    want = th.astype(F).reshape(-1, N) - f32(1e-3) * (gg / (np.abs(gg) + f32(eps)) + f32(0.01) * th.astype(F).reshape(-1, N))
    # the only rounding is the fp32 wire value of (1 - beta1) g
    assert np.max(np.abs(sh.theta - want)) <= 1e-3 * 2.0 ** -23
    assert np.allclose(sh.v, (1 - f32(0.999)) * gg * gg, rtol=1e-15, atol=0)


def test_sign_on_is_rejected():
    """A ternary Q carries no magnitude for sqrt(v) to normalise: the oracle
    refuses Decoupled AdamW with the sign on (encode and decode)."""
    L = 32 * 2
    g, th = _state(L, 2)
    sh = Shard.contiguous(L, np.zeros(L, np.float32), th)
    p = Params(scheme=RANDOM, k=32, sign=1, beta=0.9, lr=1e-3, step=0)
    with pytest.raises(ValueError):
        sh.encode(p, oracle.pad_chunks(g, L), AdamW())
    with pytest.raises(ValueError):
        sh.decode(p, [np.zeros((2, 32), np.int32)], [np.ones((2, 32))], AdamW())


def _torch_adamw(theta0, grads, lr, b1, b2, eps, wd):
    """torch.optim.AdamW in float64 over the gradient sequence: theta after
    each step and the final moments."""
    import torch

    th = torch.tensor(theta0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([th], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    thetas = []
    for g in grads:
        th.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        thetas.append(th.detach().numpy().copy())
    st = opt.state[th]
    return thetas, st["exp_avg"].numpy().copy(), st["exp_avg_sq"].numpy().copy()


@pytest.mark.parametrize("b2,eps,wd", [(0.999, 1e-8, 0.01), (0.95, 1e-3, 0.0), (0.5, 1e-6, 0.3)])
def test_first_step_equals_torch_adamw(b2, eps, wd):
    """Step 1 with every position extracted (Random n = 32), one replica and
    fp32 values: Q = fp32((1-beta1) g) and m_hat = g, so the update is
    torch.optim.AdamW's first step up to that one fp32 rounding."""
    L = 32 * 12
    g, th = _state(L, 21)
    g = (g * np.float32(1e-3)).astype(np.float32)
    lr, b1 = f32(1e-3), f32(0.9)
    ref, _, v_ref = _torch_adamw(th.astype(F), [g.astype(F)], lr, b1, f32(b2), f32(eps), f32(wd))
    w = AdamW(beta2=b2, eps=eps, weight_decay=wd)
    p = Params(scheme=RANDOM, k=32, sign=0, value_fmt=oracle.F32, beta=0.9, lr=1e-3, step=0)
    sh = Shard.contiguous(L, np.zeros(L, np.float32), th)
    idx, val, _, _ = sh.encode(p, oracle.pad_chunks(g, L), w)
    sh.decode(p, [idx], [val], w)
    assert np.allclose(sh.v.reshape(-1), v_ref, rtol=1e-14, atol=0)
    # |Q - (1-beta1) g| <= 2^-24 |Q|: the update differs by at most lr c1 2^-24 |Q|/(sqrt(v_hat)+eps)
    assert np.max(np.abs(sh.theta.reshape(-1) - ref[0])) <= float(lr) * 2.0 ** -23


@pytest.mark.parametrize("period", [2, 5, 16])
def test_diloco_moments_and_sync_step_equal_torch_adamw(period):
    """DiLoCo with period P extracts nothing on steps 0..P-2, so m and v are
    AdamW's exp_avg and exp_avg_sq there; on the sync step P-1 everything is
    extracted (Q = fp32 of AdamW's m_P) and applied with t = P.  Weight decay
    0, so the step's change of theta is AdamW's step P change (torch's theta
    moved on earlier steps, ours did not; the Adam direction does not depend
    on theta)."""
    L = 32 * 10
    rng = np.random.default_rng(30 + period)
    grads = [(rng.standard_normal(L) * 1e-3).astype(np.float32) for _ in range(period)]
    th = (rng.standard_normal(L) * 0.02).astype(np.float32)
    lr, b1, b2, eps = f32(1e-3), f32(0.9), f32(0.999), f32(1e-8)
    w = AdamW(beta2=0.999, eps=1e-8, weight_decay=0.0)
    sh = Shard.contiguous(L, np.zeros(L, np.float32), th)
    for t in range(period):
        p = Params(scheme=DILOCO, period=period, sign=0, value_fmt=oracle.F32, beta=0.9, lr=1e-3, step=t)
        if t < period - 1:
            idx, val, _, _ = sh.encode(p, oracle.pad_chunks(grads[t], L), w)
            sh.decode(p, [idx], [val], w)
            thetas, m_ref, v_ref = _torch_adamw(th.astype(F), [x.astype(F) for x in grads[:t + 1]], lr, b1, b2,
                                                 eps, 0.0)
            # fp64 on both sides, different operation order: within 1e-13 of the largest entry
            assert np.max(np.abs(sh.m.reshape(-1) - m_ref)) <= 1e-13 * np.max(np.abs(m_ref)), t
            assert np.max(np.abs(sh.v.reshape(-1) - v_ref)) <= 1e-13 * np.max(v_ref), t
            assert np.array_equal(sh.theta.reshape(-1), th.astype(F))
        else:
            before = sh.theta.copy()
            idx, val, _, _ = sh.encode(p, oracle.pad_chunks(grads[t], L), w)
            sh.decode(p, [idx], [val], w)
            thetas, m_ref, v_ref = _torch_adamw(th.astype(F), [x.astype(F) for x in grads], lr, b1, b2, eps, 0.0)
            prev = thetas[-2] if period > 1 else th.astype(F)
            step_ref = thetas[-1] - prev
            step = (sh.theta - before).reshape(-1)
            assert np.max(np.abs(sh.v.reshape(-1) - v_ref)) <= 1e-13 * np.max(v_ref)
            assert np.all(sh.m == 0.0)
            # Q = fp32(m_P): relative rounding 2^-24 of each step element
            assert np.max(np.abs(step - step_ref)) <= 2.0 ** -23 * np.max(np.abs(step_ref)) + 1e-18


def test_constant_gradient_recursion():
    """g constant, every slot extracted each step (m returns to 0): u_t =
    (1-beta1) g, v_t = (1 - beta2^t) g^2, and theta follows
    theta_t = theta_{t-1} - eta*(u_t/(1-beta1^t) / (|g| + eps) + wd*theta_{t-1})."""
    L = 32 * 6
    g, th0 = _state(L, 3)
    b1, b2, lr, eps, wd = f32(0.9), f32(0.999), f32(1e-3), f32(1e-8), f32(0.01)
    w = AdamW(beta2=0.999, eps=1e-8, weight_decay=0.01)
    sh = Shard.contiguous(L, np.zeros(L, np.float32), th0)
    gg = g.astype(F).reshape(-1, N)
    th = th0.astype(F).reshape(-1, N)
    for t in range(1, 6):
        p = Params(scheme=RANDOM, k=32, sign=0, value_fmt=oracle.F32, beta=0.9, lr=1e-3, step=t - 1)
        idx, val, _, _ = sh.encode(p, oracle.pad_chunks(g, L), w)
        assert np.allclose(sh.v, (1 - b2 ** t) * gg * gg, rtol=1e-13, atol=0)
        assert np.all(sh.m == 0.0)
        sh.decode(p, [idx], [val], w)
        u = (1 - b1) * gg
        th = th - lr * (u / (1 - b1 ** t) / (np.abs(gg) + eps) + wd * th)
        assert np.max(np.abs(sh.theta - th)) <= 1e-9, t  # fp32 wire values of u


def test_zero_gradient_only_decays():
    L = 32 * 4
    _, th0 = _state(L, 4)
    w = AdamW(weight_decay=0.1)
    sh = Shard.contiguous(L, np.zeros(L, np.float32), th0)
    for t in range(3):
        p = Params(scheme=DCT, k=2, sign=0, value_fmt=oracle.F32, beta=0.9, lr=1e-2, step=t)
        idx, val, _, _ = sh.encode(p, np.zeros((L // N, N), np.float32), w)
        sh.decode(p, [idx], [val], w)
    want = th0.astype(F).reshape(-1, N) * (1 - f32(1e-2) * f32(0.1)) ** 3
    assert np.allclose(sh.theta, want, rtol=1e-14, atol=0)
    assert np.all(sh.v == 0.0) and np.all(sh.m == 0.0)


def test_first_moment_feedback_invariant():
    """u = beta1*m + (1-beta1)*g = m' + q (DCT extraction of the first moment)."""
    L = 32 * 16
    g, _ = _state(L, 5)
    m0 = np.random.default_rng(6).standard_normal(L).astype(np.float32)
    sh = Shard.contiguous(L, m0, np.zeros(L, np.float32))
    p = Params(scheme=DCT, k=3, sign=0, value_fmt=oracle.F32, beta=0.9)
    _, _, q, _ = sh.encode(p, oracle.pad_chunks(g, L), AdamW())
    u = f32(0.9) * m0.astype(F).reshape(-1, N) + (1 - f32(0.9)) * g.astype(F).reshape(-1, N)
    assert np.max(np.abs(sh.m + q - u)) <= 1e-15 * np.max(np.abs(u)) * 4


def test_diloco_between_syncs_leaves_theta_untouched():
    L = 32 * 4
    g, th0 = _state(L, 7)
    w = AdamW(weight_decay=0.5)
    sh = Shard.contiguous(L, np.zeros(L, np.float32), th0)
    p = Params(scheme=DILOCO, period=4, step=1, sign=0, value_fmt=oracle.F32)
    idx, val, _, _ = sh.encode(p, oracle.pad_chunks(g, L), w)
    sh.decode(p, [idx], [val], w)
    assert np.array_equal(sh.theta, th0.astype(F).reshape(-1, N))
    assert np.allclose(sh.m, (1 - f32(0.9)) * g.astype(F).reshape(-1, N), rtol=1e-15, atol=0)
