"""The benchmark's algorithmic-bytes model against the pages' cache sizes."""

import bench


def test_kv_elements_match_the_pages(golden):
    rows = {r[0]: r[1:] for r in golden("kv_cache_elements.txt")}
    for label in ("sigma15b", "gqa_std"):
        n_k, d_k, n_v, d_v, elems = map(int, rows[label])
        assert bench.kv_elements_per_token(n_k, d_k, n_v, d_v) == elems
    sigma = bench.kv_elements_per_token(*map(int, rows["sigma15b"][:4]))
    gqa = bench.kv_elements_per_token(*map(int, rows["gqa_std"][:4]))
    # Eq. (2): the reduction rate tends to (32 - 20) / 32 = 37.5%.
    assert abs(100.0 * (gqa - sigma) / gqa - float(rows["reduction"][0])) < 1e-12


def test_byte_ratio_bounds_of_the_workloads():
    # Symmetric / asymmetric bytes per token for the 32k and 64k workloads.
    asym = bench.kv_elements_per_token(4, 64, 16, 128)
    asym128 = bench.kv_elements_per_token(4, 128, 16, 128)
    sym = bench.kv_elements_per_token(16, 128, 16, 128)
    assert (asym * 2, asym128 * 2, sym * 2) == (4608, 5120, 8192)
    assert abs(sym / asym128 - 1.6) < 1e-12   # exactly the pages' 37.5%
