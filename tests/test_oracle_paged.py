"""Pin for the paged-cache addressing: gathering pages by the block table is
the inverse of scattering a contiguous cache into pages, checked element by
element against the addressing rule (slot j % P of page table[b, j // P])."""
import numpy as np

from oracle import cache as ocache


def test_gather_is_the_addressing_rule_and_inverts_a_scatter():
    rng = np.random.default_rng(0)
    B, Hkv, P, npp, extra = 3, 2, 4, 5, 7
    pages = B * npp + extra
    table = rng.permutation(pages)[:B * npp].reshape(B, npp).astype(np.int32)
    cont = rng.integers(0, 255, (B, Hkv, npp * P, 6)).astype(np.uint8)
    pool = np.full((pages, Hkv, P, 6), 0xAB, np.uint8)
    for b in range(B):
        for j in range(npp * P):
            pool[table[b, j // P], :, j % P] = cont[b, :, j]
    got = ocache.gather_pages(pool, table, P)
    assert np.array_equal(got, cont)
    # per-tile arrays: 2 entries per page
    vs = rng.integers(0, 255, (pages, Hkv, 2)).astype(np.uint8)
    g = ocache.gather_pages(vs, table, P, rows_per_page=2)
    for b in range(B):
        for t in range(npp * 2):
            assert np.array_equal(g[b, :, t], vs[table[b, t // 2], :, t % 2])
