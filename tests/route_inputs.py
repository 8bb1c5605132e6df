"""Adversarial inputs for the routed path (test helper): data on which the
FP16 and the low-precision score routes differ by far more than the
tolerance, so that any group taken on the wrong route is visible in the
output.  Inputs only; no attention arithmetic lives here."""
import numpy as np

# scales that spread the FP16 scores over a few units (INT8 scores are 0)
ADV_SCALE = {"int8": 0.0883883461356163, "fp8": 0.2}


def adversarial(rng, heads, qsl, ksl, d, lowp, lens=None):
    """q, k, v such that the INT8 (or FP8) score of every (row, key) is exactly
    0 while the FP16 score is scale * a_i * c_j with |a_i c_j| of several
    units, and v is +-1 per (key tile, channel).

    k[j] = (127, c_j, 0, ...): amax 127 gives s_k = 1 (INT8) and codes
    (127, 0, ...) for |c_j| < 0.5 (FP8: s_k = 127/448, and |c_j| below
    2^-10 * 127/448 rounds to the e4m3 zero).  q[i] = (0, a_i, noise): the
    query code of channel 0 is 0, so the low-precision dot is 0."""
    n_kv, n_q = heads[1], heads[0]
    if lens is None:
        kshape, qshape = (1, n_kv, ksl, d), (1, n_q, qsl, d)
    else:
        T = sum(lens)
        kshape, qshape = (n_kv, T, d), (n_q, T, d)
    k = np.zeros(kshape, dtype=np.float16)
    k[..., 0] = 127.0
    if lowp == "fp8":
        k[..., 1] = rng.uniform(-2.6e-4, 2.6e-4, kshape[:-1]).astype(np.float16)
        amag = (30000.0, 60000.0)
    else:
        k[..., 1] = rng.uniform(-0.49, 0.49, kshape[:-1]).astype(np.float16)
        amag = (100.0, 140.0)
    q = (rng.standard_normal(qshape) * 0.5).astype(np.float16)
    q[..., 0] = 0.0
    q[..., 1] = (rng.uniform(*amag, qshape[:-1]) * rng.choice([-1.0, 1.0], qshape[:-1])).astype(np.float16)
    n_keys = kshape[-2]
    tile_sign = rng.choice([-1.0, 1.0], (n_kv, -(-n_keys // 64), d))
    vt = np.repeat(tile_sign, 64, axis=1)[:, :n_keys]
    v = (vt + 0.05 * rng.standard_normal((n_kv, n_keys, d))).astype(np.float16)
    v = v.reshape(kshape)
    return q, k, v
