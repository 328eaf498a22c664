"""The library's host Adam step (zi_adam_update) against the oracle's fp64
Adam, on the CPU: no GPU is involved in this entry point."""
import numpy as np
import pytest

import oracle
from offload_memory_centric_amd import zi

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
# the library takes its hyperparameters in fp32: the oracle gets the same values
HP32 = {k: float(np.float32(x)) for k, x in HP.items()}


def hparams(**kw):
    d = dict(HP)
    d.update(kw)
    return zi.zi_adam_hparams(**d)


def weights16(n, dtype, seed):
    """n 16-bit weights ~ N(0, 0.02) and their exact fp32 values."""
    rng = np.random.default_rng(seed)
    bits = oracle.encode(rng.normal(0.0, 0.02, n), dtype)
    return bits, oracle.decode(bits, dtype).astype(np.float32)


def grads(n, dtype, grad_f32, seed):
    rng = np.random.default_rng(seed)
    g = rng.normal(0.0, 1e-2, n) * rng.choice([1e-3, 1.0, 30.0], n)
    if grad_f32:
        g32 = g.astype(np.float32)
        return g32, g32.astype(np.float64)
    bits = oracle.encode(g, dtype)
    return bits, oracle.decode(bits, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("grad_f32", [0, 1])
def test_steps_match_the_oracle(dtype, grad_f32):
    n = 10007  # not a multiple of the 8-wide vector or the 64-element blocks
    code = zi.DTYPE_CODES[dtype]
    _, master = weights16(n, dtype, 1)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    w = np.zeros(n, np.uint16)
    om, omm, ov = master.astype(np.float64), np.zeros(n), np.zeros(n)
    hp = hparams()
    for step in range(1, 6):
        g, g64 = grads(n, dtype, grad_f32, 10 + step)
        zi.zi_adam_update(hp, code, grad_f32, step, n, g, master, m, v, w, threads=3)
        om, omm, ov = oracle.adam_step(om, omm, ov, g64, step, **HP32)
    # fp32 arithmetic against fp64: a few roundings per step
    assert np.max(np.abs(master - om)) <= 1e-7, np.max(np.abs(master - om))
    assert np.max(np.abs(m - omm)) <= 1e-6 * np.max(np.abs(omm))
    assert np.max(np.abs(v - ov)) <= 1e-6 * np.max(np.abs(ov))
    # w is the 16-bit rounding of the library's own master, bit for bit ...
    assert np.array_equal(w, oracle.encode(master.astype(np.float64), dtype))
    # ... and of the oracle's master except where the two masters straddle a tie
    want = oracle.encode(om, dtype)
    bad = np.nonzero(w != want)[0]
    if bad.size:
        lo, hi = oracle.decode(w[bad], dtype), oracle.decode(want[bad], dtype)
        assert np.all(np.abs(om[bad] - 0.5 * (lo + hi)) <= 2e-7), "w off the oracle away from a tie"
        assert bad.size <= n // 1000


def test_vector_and_scalar_code_agree_bit_for_bit():
    # one call runs the 8-wide code; single-element calls run the scalar code
    n = 1000
    for dtype in ("f16", "bf16"):
        code = zi.DTYPE_CODES[dtype]
        _, master0 = weights16(n, dtype, 2)
        g, _ = grads(n, dtype, 0, 3)
        state = []
        for single in (False, True):
            master, m, v = master0.copy(), np.full(n, 1e-4, np.float32), np.full(n, 1e-6, np.float32)
            w = np.zeros(n, np.uint16)
            if single:
                for i in range(n):
                    zi.zi_adam_update(hparams(), code, 0, 7, 1, g[i:], master[i:], m[i:], v[i:], w[i:], threads=1)
            else:
                zi.zi_adam_update(hparams(), code, 0, 7, n, g, master, m, v, w, threads=1)
            state.append((master, m, v, w))
        for a, b in zip(*state):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b.view(np.uint32) if b.dtype == np.float32 else b)


def test_thread_count_does_not_change_results():
    n = 100003
    _, master0 = weights16(n, "f16", 4)
    g, _ = grads(n, "f16", 0, 5)
    out = []
    for threads in (1, 4, 7):
        master, m, v, w = master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
        zi.zi_adam_update(hparams(), zi.ZI_F16, 0, 1, n, g, master, m, v, w, threads=threads)
        out.append(master.view(np.uint32).copy())
    assert np.array_equal(out[0], out[1]) and np.array_equal(out[0], out[2])


@pytest.mark.parametrize("bad", [dict(step=0), dict(hp=dict(beta1=1.0)), dict(hp=dict(beta2=-0.1)),
                                 dict(hp=dict(eps=-1.0)), dict(hp=dict(lr=float("inf"))), dict(dtype=3),
                                 dict(count=-1), dict(grad_f32=2), dict(null=True)])
def test_bad_arguments_are_rejected(bad):
    n = 16
    master, m, v = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    w = np.zeros(n, np.uint16)
    g = np.zeros(n, np.uint16)
    keep = master.copy()
    with pytest.raises(zi.ZiError) as e:
        zi.zi_adam_update(hparams(**bad.get("hp", {})), bad.get("dtype", zi.ZI_F16), bad.get("grad_f32", 0),
                          bad.get("step", 1), bad.get("count", n), None if bad.get("null") else g,
                          master, m, v, w)
    assert e.value.status == zi.ZI_ERR_ARG
    assert np.array_equal(master, keep)


def test_empty_update_is_a_no_op():
    zi.zi_adam_update(hparams(), zi.ZI_F16, 0, 1, 0, None, None, None, None, None)
