"""Oracle containers shared by the GPU test modules (one encode per layer
per session). Test-only: it calls the CPU oracle."""

import oracle as O

_cache = {}


def oracle_container(name, gen):
    """(layer bytes, oracle container) for the generator ``gen``, cached by name."""
    if name not in _cache:
        x = gen()
        _cache[name] = (x, O.encode_layer(x))
    return _cache[name]
