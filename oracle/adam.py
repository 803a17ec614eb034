"""Oracle O5: Adam on one rank's fp32 master partition.
TEST INFRASTRUCTURE ONLY.

[Megatron DP] "分布式优化器" and "通信模式" sections: after the reduce-scatter
each card updates only its own 1/DP slice of the parameters with its fp32
master copy; the optimizer state per parameter is fp32 master, Adam
momentum m and Adam variance v ("朴素 DP 的致命浪费" table).  The pages give no
formula, so the update is the textbook one ([Adam] Algorithm 1), with no
weight decay and the step t counted from 1:

    m' = b1*m + (1-b1)*g
    v' = b2*v + (1-b2)*(g*g)
    mh = m' / (1 - b1^t)
    vh = v' / (1 - b2^t)
    theta' = theta - (lr*mh) / (sqrt(vh) + eps)

Reading of the precision: the hyper-parameters are real numbers given by the
user (float64 here); each constant derived from them -- b1, 1-b1, b2, 1-b2,
1-b1^t, 1-b2^t, lr, eps -- is formed in float64 and rounded once to fp32.
Every operation on the per-element state is then one fp32 operation,
evaluated left to right as written.
"""

import numpy as np


def constants(lr, beta1, beta2, eps, step):
    """The fp32 constants of one step, each formed in float64 and rounded
    once: (b1, 1-b1, b2, 1-b2, 1-b1^t, 1-b2^t, lr, eps)."""
    f = np.float32
    b1, b2 = float(beta1), float(beta2)
    return (f(b1), f(1.0 - b1), f(b2), f(1.0 - b2),
            f(1.0 - b1 ** step), f(1.0 - b2 ** step), f(lr), f(eps))


def bias_corrections(beta1, beta2, step):
    """(1 - b1^t, 1 - b2^t) formed in float64, rounded to fp32."""
    c = constants(0.0, beta1, beta2, 0.0, step)
    return c[4], c[5]


def adam_oracle(grad, master, m, v, lr, beta1, beta2, eps, step):
    """Returns (master', m', v') as new float32 arrays."""
    f = np.float32
    g = np.asarray(grad, f)
    th = np.asarray(master, f)
    m0 = np.asarray(m, f)
    v0 = np.asarray(v, f)
    b1, c1, b2, c2, bc1, bc2, lr32, eps32 = constants(lr, beta1, beta2, eps,
                                                      step)
    m1 = np.add(np.multiply(b1, m0, dtype=f),
                np.multiply(c1, g, dtype=f), dtype=f)
    gg = np.multiply(g, g, dtype=f)
    v1 = np.add(np.multiply(b2, v0, dtype=f),
                np.multiply(c2, gg, dtype=f), dtype=f)
    mh = np.divide(m1, bc1, dtype=f)
    vh = np.divide(v1, bc2, dtype=f)
    denom = np.add(np.sqrt(vh, dtype=f), eps32, dtype=f)
    upd = np.divide(np.multiply(lr32, mh, dtype=f), denom, dtype=f)
    th1 = np.subtract(th, upd, dtype=f)
    return th1, m1, v1


def adam_oracle_f64(grad, master, m, v, lr, beta1, beta2, eps, step):
    """The same update carried out in float64 from the same fp32 state and
    the float64 hyper-parameters (a sanity twin: the fp32 oracle must stay
    within tolerance of it)."""
    d = np.float64
    g = np.asarray(grad, np.float32).astype(d)
    th = np.asarray(master, np.float32).astype(d)
    m0 = np.asarray(m, np.float32).astype(d)
    v0 = np.asarray(v, np.float32).astype(d)
    b1, b2, lr64, eps64 = d(beta1), d(beta2), d(lr), d(eps)
    m1 = b1 * m0 + (1.0 - b1) * g
    v1 = b2 * v0 + (1.0 - b2) * g * g
    mh = m1 / (1.0 - b1 ** step)
    vh = v1 / (1.0 - b2 ** step)
    th1 = th - lr64 * mh / (np.sqrt(vh) + eps64)
    return th1, m1, v1
