"""Analytic theta-bundle sizes ("Compression" page, "Theta-bundle size: the
sharing headroom" and "Where the bytes go"; "Quality" page, "The coherence
frontier" for the footprint definition).

All counts are elements; bytes use 4 bytes per element (float32), the dtype
the pages use for this analysis.  For one family with out dim N, in dim K,
rank r, G bands and L layers:
    W0: G * N * K,  s: L * N,  U: L * N * r,  V: L * K * r
and the dense projections take L * N * K.  Footprint = theta / dense.
"""


def family_counts(N, K, r, num_layers, num_bands):
    return {"W0": num_bands * N * K, "s": num_layers * N,
            "U": num_layers * N * r, "V": num_layers * K * r,
            "dense": num_layers * N * K}


def bundle_counts(shapes, rank, num_layers, num_bands):
    """shapes: iterable of (N, K), one per family."""
    tot = {"W0": 0, "s": 0, "U": 0, "V": 0, "dense": 0}
    for N, K in shapes:
        for k, v in family_counts(N, K, rank, num_layers, num_bands).items():
            tot[k] += v
    tot["theta"] = tot["W0"] + tot["s"] + tot["U"] + tot["V"]
    return tot


def bundle_mb(shapes, rank, num_layers, num_bands, bytes_per_elem=4):
    c = bundle_counts(shapes, rank, num_layers, num_bands)
    return {k: v * bytes_per_elem / 1e6 for k, v in c.items()}
