"""Hand-built fp16 groups that stress a min/max 4-bit quantizer (inputs only)."""
import numpy as np

G = 64


def adversarial_groups() -> np.ndarray:
    """Concatenated 64-element fp16 groups: constant, two-valued, extreme range,
    subnormal, signed zeros, exact ties, and huge/tiny mixtures."""
    rng = np.random.default_rng(1234)
    groups = []
    groups.append(np.zeros(G))
    groups.append(np.full(G, -0.0))
    groups.append(np.where(np.arange(G) % 2, 0.0, -0.0))
    groups.append(np.full(G, 3.25))
    groups.append(np.where(np.arange(G) % 3 == 0, 1.0, -1.0))
    groups.append(np.where(np.arange(G) % 5 == 0, 65504.0, -65504.0))
    groups.append(np.linspace(-65504.0, 65504.0, G))
    groups.append(rng.uniform(-1, 1, G) * 2.0 ** -20)           # subnormal values
    groups.append(np.arange(G) * 2.0 ** -24)                    # subnormal ladder
    groups.append(np.concatenate([[2.0 ** -24], np.zeros(G - 1)]))  # scale underflows to zero
    groups.append(np.concatenate([[65504.0], np.full(G - 1, 2.0 ** -24)]))
    groups.append(np.arange(G) % 16)
    s, mn = 2.0 ** -6, -0.25
    k = np.arange(15)
    v = np.concatenate([[mn, mn + 15 * s], mn + (k + 0.5) * s])
    groups.append(np.concatenate([v, np.full(G - v.size, mn)]))  # exact ties
    for e in range(-12, 12, 3):                                  # ties at other scales
        s = 2.0 ** e
        mn = -3 * s
        v = np.concatenate([[mn, mn + 15 * s], mn + (k + 0.5) * s])
        groups.append(np.concatenate([v, rng.uniform(mn, mn + 15 * s, G - v.size)]))
    for _ in range(40):
        scale = 10.0 ** rng.uniform(-6, 4)
        groups.append(rng.standard_normal(G) * scale + rng.standard_normal() * scale * 10)
    x = np.concatenate(groups)
    with np.errstate(over="ignore"):
        x = np.clip(x, -65504.0, 65504.0).astype(np.float16)
    return x
