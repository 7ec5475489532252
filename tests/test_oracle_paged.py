"""Pins of the paged plane layout (reading R24: the pages fix no memory
layout; a paged cache stores the same 64-position tiles as the contiguous
one, [page][g][tile] instead of [b][g][t]).

* With one KV head and the table page = b * tiles + t, the pool is the
  contiguous plane byte for byte.
* Hand-placed tiles land where the layout says, for several KV heads.
* Scatter then gather is the identity on every tile a table names.
* A whole oracle cache survives the round trip through a shuffled pool, and
  attention over the gathered planes equals attention over the original."""

import numpy as np
import pytest

import workloads
from oracle import (OracleCache, decode_reference, pages_to_contiguous, contiguous_to_pages,
                    padded_row_bytes)
from oracle.blockquant import TILE, v_tile_bytes, bf16_bits_to_f32


def test_identity_table_one_head_is_contiguous():
    B, tiles, ts = 3, 5, 7
    rng = np.random.default_rng(0)
    plane = rng.integers(0, 256, size=(B, 1, tiles * ts), dtype=np.uint8)
    table = np.arange(B * tiles).reshape(B, tiles)
    pool = contiguous_to_pages(plane, table, B * tiles, ts)
    assert np.array_equal(pool.reshape(-1), plane.reshape(-1))
    assert np.array_equal(pages_to_contiguous(plane.reshape(-1), table, 1, ts), plane)


def test_hand_placed_tiles():
    # pool of 4 pages x 2 heads x 3-element tiles, element value = 100*page + 10*g + i
    H, ts = 2, 3
    pool = np.array([[[100 * p + 10 * g + i for i in range(ts)] for g in range(H)]
                     for p in range(4)], dtype=np.int32)
    table = np.array([[2, 0], [3, -1]])
    got = pages_to_contiguous(pool, table, H, ts)
    # sequence 0: tile 0 from page 2, tile 1 from page 0
    assert list(got[0, 1]) == [210, 211, 212, 10, 11, 12]
    assert list(got[0, 0]) == [200, 201, 202, 0, 1, 2]
    # sequence 1: tile 0 from page 3, tile 1 unmapped (zero)
    assert list(got[1, 0]) == [300, 301, 302, 0, 0, 0]
    assert list(got[1, 1]) == [310, 311, 312, 0, 0, 0]


def test_scatter_gather_round_trip():
    rng = np.random.default_rng(1)
    B, H, tiles, ts, P = 4, 3, 6, 11, 40
    plane = rng.integers(0, 65536, size=(B, H, tiles * ts), dtype=np.uint16)
    table = rng.permutation(P)[: B * tiles].reshape(B, tiles)
    pool = contiguous_to_pages(plane, table, P, ts)
    assert np.array_equal(pages_to_contiguous(pool, table, H, ts), plane)
    # pages no entry names stay zero
    unused = sorted(set(range(P)) - set(table.reshape(-1).tolist()))
    assert not pool[unused].any()


@pytest.mark.parametrize("d,kb,vb,km,T", [(64, 4, 8, False, 0), (128, 8, 4, False, 16),
                                         (256, 5, 4, True, 0)])
def test_oracle_cache_through_a_shuffled_pool(d, kb, vb, km, T):
    B, H, n, max_ctx = 2, 2, 150, 200
    orc = OracleCache(B, H, d, kb, vb, T, max_ctx, k_min=km)
    k = workloads.adversarial_numpy(1, (B, n, H, d))
    v = workloads.adversarial_numpy(2, (B, n, H, d))
    orc.append(k, v, [0, 0])
    want = orc.physical()
    tiles = (max_ctx + TILE - 1) // TILE
    P = B * tiles + 5
    table = np.random.default_rng(3).permutation(P)[: B * tiles].reshape(B, tiles)
    sizes = {"k_codes": TILE * padded_row_bytes(d, kb), "v_codes": v_tile_bytes(d, vb),
             "k_scales": TILE * (d // 32) * (2 if km else 1), "v_scales": TILE * (d // 32)}
    got = dict(want)
    for key, ts in sizes.items():
        flat = want[key].reshape(B, H, -1)
        pool = contiguous_to_pages(flat, table, P, ts)
        back = pages_to_contiguous(pool, table, H, ts)
        assert np.array_equal(back, flat), key
        got[key] = back.reshape(want[key].shape)
    q = workloads.adversarial_numpy(9, (B, 2 * H, d))
    a = decode_reference(want, bf16_bits_to_f32(q), [n, n], H, d, kb, vb, T, k_min=km)
    b = decode_reference(got, bf16_bits_to_f32(q), [n, n], H, d, kb, vb, T, k_min=km)
    assert np.array_equal(a, b)
