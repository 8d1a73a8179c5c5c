"""Host checks of the kernels' LDS layouts (no GPU).

The kernels' LDS addressing is restated here from the sources and checked
against two properties:
  * the direct HBM -> LDS tile loads (PaddedTileDma in common.hpp) put every
    16-byte chunk of every row where the reads expect it and never write outside
    the tile's whole-KB allocation; only slots in the slack past the last row
    fetch bytes beyond the tile's rows;
  * the reads are free of bank conflicts under the LDS model the counters
    confirm on gfx950: 64 banks of 4 bytes, a 16-byte read served 16 lanes per
    pass and an 8-byte (transposed) read 32 lanes per pass. Under this model the
    backward's former layout (rows padded by 16, natural order) is 2-way
    conflicted, which the counters showed as 38-40 % of LDS-active cycles.
The layouts checked: the prefill's XOR-swizzled 256-byte rows (prefill_bf16.hip,
D = 128, and V at D_qk = 192), its 384-byte K rows at D_qk = 192, its padded rows
at D = 64, the backward's (D + 8)-element rows read in the perm16 row order
(backward_bf16.hip), and the fp32 kernels' padded rows (prefill_f32.hip,
backward_f32.hip), whose 4-byte operand reads are served 64 lanes per pass."""
import pytest


def banks_max(addrs, width):
    """Largest number of accesses that one bank gets from one pass of lanes."""
    count = {}
    for a in addrs:
        for w in range(width // 4):
            b = (a // 4 + w) % 64
            count[b] = count.get(b, 0) + 1
    return max(count.values())


def row_read_passes(row_addr, nrows, nchunks):
    """16-byte reads of chunk c of rows r0 + l32 (l32 < 32) in lane half h:
    yields each pass of 16 lanes as a list of byte addresses."""
    for r0 in range(0, nrows, 32):
        for c in range(nchunks):
            for lanes in (range(0, 16), range(16, 32)):
                yield [row_addr(r0 + l, c) for l in lanes]


def tr_read_passes(addr):
    """ds_read_b64_tr_b16 as the PV / dV / dK / dQ products issue it: lane
    16 * gg + L reads accumulator row 8 * x + 4 * (gg // 2) + L // 4 (of a
    16-row step) at column 16 * (gg % 2) + 4 * (L % 4) of a 32-column block.
    Yields each half wave's byte addresses for every (step, x, column block)."""
    for step in range(2):
        for x in range(2):
            for mt in range(2):
                for half in range(2):
                    out = []
                    for lane in range(32 * half, 32 * half + 32):
                        gg, L = lane >> 4, lane & 15
                        rho = 16 * step + 8 * x + 4 * (gg >> 1) + (L >> 2)
                        col = 32 * mt + 16 * (gg & 1) + 4 * (L & 3)
                        out.append(addr(rho, col))
                    yield out


# ---- PaddedTileDma --------------------------------------------------------------

def padded_tile_dma_map(rows, row_bytes, stride, nw):
    """LDS byte -> global byte of the tile, as PaddedTileDma::init / issue compute it.
    The LDS tile is allocated in whole KB (padded_tile_bytes); slots past the tile's
    rows land in that slack and fetch the next global rows (clamped by the kernel)."""
    alloc = (rows * stride + 1023) // 1024 * 1024
    pieces = alloc // 1024
    per = (pieces + nw - 1) // nw
    lds = {}
    for wave in range(nw):
        for q in range(per):
            j = wave + q * nw
            if j >= pieces:
                continue
            for lane in range(64):
                p = j * 1024 + lane * 16
                row, within = divmod(p, stride)
                off = row * row_bytes + (within if within < row_bytes else within - row_bytes)
                assert p not in lds and p + 16 <= alloc
                assert 0 <= off and (row >= rows or off + 16 <= rows * row_bytes)
                lds[p] = off
    assert len(lds) == pieces * 64
    return lds


@pytest.mark.parametrize("rows,row_bytes,stride", [
    (128, 128, 144), (128, 128, 192),    # prefill D = 64: K, V
    (96, 384, 400),                      # a tile that is not whole KB (37.5 KB): slack
    (128, 256, 272),                     # dQ kernel D = 128: K and V
    (64, 256, 272), (64, 128, 144),      # dK/dV kernel Q and dO, D = 128 and 64
    # fp32 kernels (4-byte elements): prefill 32 x 32 shape, K and V at D = 128 and 64
    (64, 512, 528), (64, 512, 544), (128, 256, 272), (128, 256, 288),
    # prefill 16 x 16 shape (V padded by 4), backward dQ tiles and dK/dV query tiles
    (128, 256, 272), (32, 512, 528), (64, 512, 528),
])
def test_padded_tile_dma_places_every_chunk(rows, row_bytes, stride):
    """Every 16-byte chunk of every row lands at its row's LDS offset."""
    lds = padded_tile_dma_map(rows, row_bytes, stride, 8)
    for r in range(rows):
        for c in range(0, row_bytes, 16):
            assert lds[r * stride + c] == r * row_bytes + c


# ---- prefill, D = 128: XOR-swizzled 256-byte rows ------------------------------

def swz(r):
    x = r & 7
    return ((((x & 3) << 1) | (x >> 2)) << 1) | ((r >> 3) & 1)


def test_prefill_swizzle_is_a_permutation_of_each_row():
    for r in range(128):
        assert sorted(c ^ swz(r) for c in range(16)) == list(range(16))


def test_prefill_swizzle_reads_are_conflict_free():
    def k_addr(r, c):                       # chunk c of K row r
        return r * 256 + 16 * (c ^ swz(r))

    def v_addr(rho, col):                   # element col of V row rho, 8-byte reads
        c, within = divmod(2 * col, 16)
        return rho * 256 + 16 * (c ^ swz(rho)) + within

    assert max(banks_max(p, 16) for p in row_read_passes(k_addr, 128, 16)) == 1
    assert max(banks_max(p, 8) for p in tr_read_passes(v_addr)) == 1


@pytest.mark.parametrize("stride,kind", [(144, "row"), (192, "tr")])
def test_prefill_padded_rows_are_conflict_free(stride, kind):
    if kind == "row":   # K rows of D = 64 (144 B)
        worst = max(banks_max(p, 16) for p in row_read_passes(lambda r, c: r * stride + 16 * c, 96, stride // 16 - 1))
    else:               # V rows padded by 32 elements, read transposed
        worst = max(banks_max(p, 8) for p in tr_read_passes(lambda rho, col: rho * stride + 2 * col))
    assert worst == 1


# ---- prefill, D_qk = 192: 384-byte K rows, low three chunk bits XORed -----------

def kswz(r):
    return (r >> 1) & 7


def test_prefill_wide_k_tile_loads_and_reads():
    """The 1 KB direct loads of a 128-key tile of 384-byte K rows (6 per wave, each
    lane's global offset precomputed) fill every slot with the chunk the reads take:
    chunk 2 s + h of row krow0 + l32 at lane base kra[4 buf + s % 4] + 128 (s / 4)
    + krow0 * 384, an immediate offset below 64 KB. The reads are conflict-free."""
    rowb, bk, nw, nik = 384, 128, 8, 6
    lds = {}
    for wave in range(nw):
        for q in range(nik):
            for lane in range(64):
                b = 1024 * (wave * nik + q) + 16 * lane
                row, slot = b // rowb, (b % rowb) // 16
                lds[b] = row * rowb + 16 * (slot ^ kswz(row))
    assert sorted(lds) == list(range(0, bk * rowb, 16)) and sorted(lds.values()) == sorted(lds)

    def addr(krow0, s, l32, h):
        return l32 * rowb + 16 * ((2 * (s & 3) + h) ^ kswz(l32)) + 128 * (s >> 2) + krow0 * rowb

    for krow0 in range(0, bk, 32):
        for s in range(12):
            for l32 in range(32):
                for h in range(2):
                    a = addr(krow0, s, l32, h)
                    assert a - l32 * rowb - 16 * ((2 * (s & 3) + h) ^ kswz(l32)) < 65536
                    assert lds[a] == (krow0 + l32) * rowb + 16 * (2 * s + h)
            for h in range(2):
                for half in range(2):
                    assert banks_max([addr(krow0, s, l, h) for l in range(16 * half, 16 * half + 16)], 16) == 1


# ---- backward: (D + 8)-element rows read in the perm16 order -------------------

def perm16(r):
    return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3)


def test_perm16_is_an_involution_within_16_row_blocks():
    for r in range(256):
        assert perm16(perm16(r)) == r and perm16(r) // 16 == r // 16


@pytest.mark.parametrize("d", [64, 128])
def test_backward_row_order_is_conflict_free(d):
    stride = 2 * (d + 8)

    def row_addr(rho, c):                   # accumulator row rho reads LDS row perm16(rho)
        return perm16(rho) * stride + 16 * c

    def tr_addr(rho, col):
        return perm16(rho) * stride + 2 * col

    assert max(banks_max(p, 16) for p in row_read_passes(row_addr, 64, d // 8)) == 1
    assert max(banks_max(p, 8) for p in tr_read_passes(tr_addr)) == 1


def test_backward_former_layout_was_conflicted():
    """Rows padded by 16 elements in natural order: 2-way on both read kinds."""
    stride = 2 * (128 + 16)
    assert max(banks_max(p, 16) for p in row_read_passes(lambda r, c: r * stride + 16 * c, 64, 16)) == 2
    assert max(banks_max(p, 8) for p in tr_read_passes(lambda rho, col: rho * stride + 2 * col)) == 2


def test_backward_tr_read_rows_match_the_kernels_expression():
    """backward_bf16.hip forms the LDS row of a transposed read directly as
    16 * t2 + 4 * (L / 4) + 2 * x + gg / 2."""
    for t2 in range(2):
        for x in range(2):
            for lane in range(64):
                gg, L = lane >> 4, lane & 15
                rho = 16 * t2 + 8 * x + 4 * (gg >> 1) + (L >> 2)
                assert perm16(rho) == 16 * t2 + 4 * (L >> 2) + 2 * x + (gg >> 1)


def test_backward_mask_offsets_match_perm16():
    """Element i of lane half h holds accumulator row 8 * (i / 4) + 4 * h + i % 4;
    the masks compare its row's offset, perm16 of that, written out per element."""
    for h in range(2):
        for i in range(16):
            rho = 8 * (i >> 2) + 4 * h + (i & 3)
            assert perm16(rho) == 16 * (i >> 3) + 4 * (i & 3) + 2 * ((i >> 2) & 1) + h


# ---- fp32 kernels: rows padded by 4 floats (V by 8 with 32 x 32 products) --------

def f32_row_read_passes(M, stride, d):
    """16-byte operand reads of the fp32 products: lane L reads floats g d / G + 4 c
    .. + 3 of row L % M (G = 64 / M lane groups, g = L / M); passes of 16 lanes."""
    G = 64 // M
    for c in range(d // G // 4):
        for p in range(4):
            yield [4 * ((lane % M) * stride + (lane // M) * (d // G) + 4 * c) for lane in range(16 * p, 16 * p + 16)]


def f32_col_read_lanes(M, stride, d, step):
    """4-byte operand reads of the second products: lane L reads column L % M (+ M
    per output tile) of row 4 (L / M) + (step / 4) 4 G + step % 4; one pass of 64."""
    G = 64 // M
    for mt in range(d // M):
        row = lambda lane: 4 * (lane // M) + (step >> 2) * 4 * G + (step & 3)
        yield [4 * (row(lane) * stride + lane % M + M * mt) for lane in range(64)]


@pytest.mark.parametrize("M", [32, 16])
@pytest.mark.parametrize("d", [64, 128])
def test_f32_prefill_reads_are_conflict_free(M, d):
    ks, vs = d + 4, d + (8 if M == 32 else 4)
    assert max(banks_max(p, 16) for p in f32_row_read_passes(M, ks, d)) == 1
    for step in range(M * M // 64):
        assert max(banks_max(p, 4) for p in f32_col_read_lanes(M, vs, d, step)) == 1


def test_f32_prefill_v_padding_must_follow_the_shape():
    """Rows padded by 8 with 16 x 16 products (lane groups 32 banks apart, four of
    them) or by 4 with 32 x 32 ones (two groups 16 banks apart, 32 columns each)
    would be 2-way conflicted."""
    assert max(banks_max(p, 4) for p in f32_col_read_lanes(16, 136, 128, 0)) == 2
    assert max(banks_max(p, 4) for p in f32_col_read_lanes(32, 132, 128, 0)) == 2


@pytest.mark.parametrize("d", [64, 128])
def test_f32_backward_reads_are_conflict_free(d):
    """backward_f32.hip: 16 x 16 products only, every tile padded by 4 floats; the
    16-byte reads (S, dP) and the 4-byte reads (dQ from K; dV, dK from dO and Q)."""
    assert max(banks_max(p, 16) for p in f32_row_read_passes(16, d + 4, d)) == 1
    for step in range(4):
        assert max(banks_max(p, 4) for p in f32_col_read_lanes(16, d + 4, d, step)) == 1
