"""Host checks of the bf16 prefill's workgroup -> work-item map (no GPU).

The map is restated here from prefill_bf16.hip. When the KV heads (times batch)
are not a multiple of 8, the work list (batch, KV head, query tile heavy-first,
query head of the group) is cut into blocks of kXcdTiles query tiles and dealt in
rounds of eight, one block per XCD, in serpentine order; workgroup id b runs on XCD
b % 8. Checked: every work item is run exactly once (the rest of the padded grid
returns at once), and with causal tile weights falling linearly along a KV head
every XCD's total stays within one block's weight of the mean."""
import pytest

K_XCD_TILES = 4


def item_of(bid, bs):
    x, j = bid & 7, bid >> 3
    r = j // bs
    return (8 * r + ((7 - x) if (r & 1) else x)) * bs + j % bs


def grid_of(n_items, bs):
    nb = -(-n_items // bs)
    return 8 * (-(-nb // 8)) * bs


@pytest.mark.parametrize("B,Hkv,group,tiles", [(1, 4, 7, 32), (1, 2, 16, 64), (1, 1, 32, 64), (2, 3, 4, 17),
                                                (1, 5, 1, 3), (1, 1, 8, 1)])
def test_every_item_once(B, Hkv, group, tiles):
    n_items = B * Hkv * group * tiles
    bs = K_XCD_TILES * group
    seen = [0] * n_items
    for bid in range(grid_of(n_items, bs)):
        u = item_of(bid, bs)
        if u < n_items:
            seen[u] += 1
    assert all(c == 1 for c in seen)


@pytest.mark.parametrize("B,Hkv,group,tiles", [(1, 4, 7, 32), (1, 2, 8, 64), (1, 1, 32, 64), (1, 4, 16, 64)])
def test_xcd_totals_are_even(B, Hkv, group, tiles):
    """Causal weights: the query tile of rank t (heaviest first) costs tiles - t."""
    n_items = B * Hkv * group * tiles
    bs = K_XCD_TILES * group
    total = [0] * 8
    for bid in range(grid_of(n_items, bs)):
        u = item_of(bid, bs)
        if u < n_items:
            t = (u // group) % tiles
            total[bid & 7] += tiles - t
    mean = sum(total) / 8
    block_weight = bs * tiles
    assert max(total) - mean <= block_weight, (total, mean)
    # the contiguous eighths this replaces leave a KV-head fraction's weight spread
    eighth = -(-n_items // 8)
    total_old = [0] * 8
    for u in range(n_items):
        t = (u // group) % tiles
        total_old[u // eighth] += tiles - t
    assert max(total) < max(total_old)
