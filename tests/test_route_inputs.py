"""CPU check of the adversarial routed inputs on the oracle: flipping one
group's routing bit moves the output far past the GPU tolerance, so a
misrouted group cannot hide under it."""
import numpy as np

import workloads as W
from route_inputs import ADV_SCALE, adversarial


def test_adversarial_construction_separates_routes(orc):
    """On the oracle: with these inputs, flipping one group's bit moves some
    output element by more than 20x the tolerance (else a misroute could
    hide under it)."""
    rng = np.random.default_rng(9300)
    for lowp in ("int8", "fp8"):
        q, k, v = adversarial(rng, (2, 1), 100, 2000, 64, lowp)
        n_g = W.n_route_groups(2000, 4)
        bits = rng.random((2, n_g)) < 0.5
        sc = ADV_SCALE[lowp]
        a = orc.attn_fwd(q, k, v, scale=sc, causal=False, route=W.pack_bits(bits), tiles_per_bit=4, lowp=lowp)
        for g in (0, 3, n_g - 1):
            b2 = bits.copy()
            b2[1, g] = not b2[1, g]
            b = orc.attn_fwd(q, k, v, scale=sc, causal=False, route=W.pack_bits(b2), tiles_per_bit=4, lowp=lowp)
            assert np.abs(a - b).max() > 0.08, (lowp, g, np.abs(a - b).max())
