"""CPU model of how the trunk backward rounds dS to fp16, with and without the
power-of-two scale the kernels apply (a test of the rule, not of the kernels).

The kernels form dS = P (dP - Delta) in fp32 and round it to fp16 for the dS K
(dQ) and dS^T Q (dK) products.  Rounded as is, dS leaves fp16's range when dO is
small (a loss averaged over many tokens): subnormal below 6.1e-5, zero below
3e-8.  The kernels scale it first: per query row in the dQ kernel, 2^e with
e = 15 - exponent(||dO_i||_1 max_j |v_jd| + |Delta_i|); per key in the dK/dV
kernel, with the bound N ||v_j||_inf + Dm (N, Dm the largest ||dO_i||_1 and
|Delta_i| of the rows); both clamped to [-64, 64].  This model applies the same
rule to one causal head and compares the products against fp64.
"""
import numpy as np
import pytest

import ttt_synth as syn

S, D = 1024, 128
FP16_MAX = 65504.0


def ds_exp(x):
    _, ex = np.frexp(np.asarray(x, np.float32))
    return np.clip(15 - ex, -64, 64)


def problem(scale, seed=3):
    rng = np.random.default_rng(seed)
    q, k, v, do = (syn.round_bf16(rng.standard_normal((S, D)).astype(np.float32)) for _ in range(4))
    if scale == "mixed":
        f = (10.0 ** rng.uniform(-6, 0, (S, 1))).astype(np.float32)
    else:
        f = np.float32(scale)
    do = syn.round_bf16(do * f)
    return [x.astype(np.float64) for x in (q, k, v, do)]


def exact_parts(q, k, v, do):
    sig = 1.0 / np.sqrt(D)
    s = sig * q @ k.T
    s[np.triu_indices(S, 1)] = -np.inf
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p /= p.sum(axis=1, keepdims=True)
    o = p @ v
    delta = np.sum(do * o, axis=1)
    ds = p * (do @ v.T - delta[:, None])
    return sig, ds, delta


def model(q, k, v, do, scaled: bool):
    sig, ds, delta = exact_parts(q, k, v, do)
    f16 = lambda x: x.astype(np.float32).astype(np.float16).astype(np.float64)
    if scaled:
        n1 = np.abs(do).sum(axis=1).astype(np.float32)
        vinf = np.abs(v).max(axis=1).astype(np.float32)
        eq = ds_exp(n1 * vinf.max() + np.abs(delta).astype(np.float32))   # dQ: per row
        ek = ds_exp(n1.max() * vinf + np.abs(delta).max())                # dK: per key
        ds_q = f16(ds * np.exp2(eq)[:, None]) * np.exp2(-eq)[:, None]
        ds_k = f16(ds * np.exp2(ek)[None, :]) * np.exp2(-ek)[None, :]
        assert np.abs(ds * np.exp2(eq)[:, None]).max() < FP16_MAX
        assert np.abs(ds * np.exp2(ek)[None, :]).max() < FP16_MAX
    else:
        ds_q = ds_k = f16(ds)
    dq = sig * ds_q @ f16(k)
    dk = sig * ds_k.T @ f16(q)
    dq_x = sig * ds @ k
    dk_x = sig * ds.T @ q
    fro = lambda a, b: float(np.linalg.norm(a - b) / np.linalg.norm(b))
    return fro(dq, dq_x), fro(dk, dk_x)


@pytest.mark.parametrize("scale", [1.0, 1e-4, 1e-6, "mixed"])
def test_scaled_ds_is_accurate_at_any_dout_scale(scale):
    eq, ek = model(*problem(scale), scaled=True)
    print(f"dO*{scale}: scaled fp16 dS: dQ {eq:.1e} dK {ek:.1e}")
    assert eq <= 2e-3 and ek <= 2e-3


def test_unscaled_ds_fails_at_small_dout():
    """The failure the scale removes: at dO ~ 1e-6 plain fp16 dS misses the 1e-2 bar."""
    eq, ek = model(*problem(1e-6), scaled=False)
    print(f"dO*1e-6: unscaled fp16 dS: dQ {eq:.1e} dK {ek:.1e}")
    assert max(eq, ek) > 1e-2
    eq1, ek1 = model(*problem(1.0), scaled=False)
    assert max(eq1, ek1) <= 2e-3


def test_scale_bound_holds_for_large_dout_and_values():
    q, k, v, do = problem(1.0)
    v *= 1e3
    do *= 1e3
    eq, ek = model(q, k, v, do, scaled=True)   # asserts |2^e dS| < 65504 inside
    assert eq <= 2e-3 and ek <= 2e-3


def test_power_of_two_scale_shifts_the_exponent_exactly():
    x = np.float32([3.0e-7, 1.0, 12345.0])
    assert np.array_equal(ds_exp(x * np.float32(2.0 ** -20)), ds_exp(x) + 20)
    assert ds_exp(np.float32(0.0)) == 15 and ds_exp(np.float32(1e-30)) == 64 and ds_exp(np.float32(1e30)) == -64
