"""The kernels' closed-form index functions, evaluated on the host through
the C ABI (the same __host__ __device__ code the kernels run), against the
layouts the Shape:Stride module computes for the same maps.  This is the
"hand arithmetic against the layout algebra" gate of "cute_layouts.cu"
applied to every map the GEMM kernels rely on.
"""
import pytest

import tile_hierarchy_linear_amd as thl


def _eval(layout, n):
    return thl.thl_layout_eval(layout, range(n))


def test_map_names_are_all_known():
    names = thl.thl_kernel_index_map_names()
    for n in names:
        pts = [(0, 0)]
        params = {"xcd_remap": (8,), "grouped_tile": (4, 4, 2), "copy_source": (16,),
                  "mfma32_operand": (8,), "mm_lds_offset": (256,), "mm_copy_source": (16, 256),
                  "pair_lds_offset": (0,)}.get(n, ())
        thl.thl_kernel_index_map(n, pts, params)
    with pytest.raises(thl.ThlError):
        thl.thl_kernel_index_map("no_such_map", [(0, 0)])


@pytest.mark.parametrize("vals", [8, 16, 32])
def test_mfma_operand_map_is_the_tv_layout(vals):
    # lane l, value v -> (row l%32, k (l/32)*vals + v), as the TV layout
    # ((32,2),vals):((1,32*vals),32) onto the column-major index row + 32*k.
    tv = f"((32,2),{vals}):((1,{32 * vals}),32)"
    pts = [(l, v) for v in range(vals) for l in range(64)]
    got = thl.thl_kernel_index_map("mfma32_operand", pts, (vals,))
    want = _eval(tv, 64 * vals)
    assert [r + 32 * k for r, k in got] == want
    assert sorted(want) == list(range(64 * vals))  # every operand element once


def test_mfma_accumulator_map_is_the_tv_layout():
    tv = "((32,2),(4,4)):((32,4),(1,8))"
    pts = [(l, v) for v in range(16) for l in range(64)]
    got = thl.thl_kernel_index_map("mfma32_acc", pts)
    want = _eval(tv, 1024)
    assert [r + 32 * c for r, c in got] == want
    assert sorted(want) == list(range(1024))
    # runs of four consecutive rows per lane (vector stores along M)
    for l in range(64):
        rows = [got[v * 64 + l][0] for v in range(16)]
        for q in range(4):
            assert rows[4 * q:4 * q + 4] == list(range(rows[4 * q], rows[4 * q] + 4))


def test_small_m_operand_map_is_the_tv_layout():
    # the small-M kernel's 128-byte K unit: lane l, byte j -> (row l%16, byte
    # 64*(j/16) + 16*(l/16) + j%16), the TV layout ((16,4),(16,2)):((128,16),(1,64))
    # onto the row-major index kbyte + 128*row
    tv = "((16,4),(16,2)):((128,16),(1,64))"
    pts = [(l, j) for j in range(32) for l in range(64)]
    got = thl.thl_kernel_index_map("mfma16_operand", pts)
    want = _eval(tv, 2048)
    assert [kb + 128 * r for r, kb in got] == want
    assert sorted(want) == list(range(2048))  # every byte of 16 rows x 128 bytes once
    # each 16-byte half is contiguous and 16-byte aligned: one fp4 scale block
    # (32 elements), block 4*h + l/16 of the unit
    for l in range(64):
        for h in range(2):
            kbs = [got[(16 * h + j) * 64 + l][1] for j in range(16)]
            assert kbs == list(range(kbs[0], kbs[0] + 16)) and kbs[0] % 16 == 0
            assert kbs[0] // 16 == 4 * h + l // 16


def test_small_m_accumulator_map_is_the_tv_layout():
    tv = "((16,4),4):((16,4),1)"
    pts = [(l, v) for v in range(4) for l in range(64)]
    got = thl.thl_kernel_index_map("mfma16_acc", pts)
    want = _eval(tv, 256)
    assert [r + 16 * c for r, c in got] == want
    assert sorted(want) == list(range(256))
    for l in range(64):  # four consecutive rows of one column per lane
        rows = [got[v * 64 + l][0] for v in range(4)]
        assert rows == list(range(rows[0], rows[0] + 4)) and len({got[v * 64 + l][1] for v in range(4)}) == 1


def test_fp8_k_order_covers_each_k_once_per_row():
    for row in range(32):
        ks = sorted(k for lane in (row, row + 32) for (k, _) in
                    thl.thl_kernel_index_map("fp8_32x32_k", [(lane, j) for j in range(32)]))
        assert ks == list(range(64))


def test_tr16_source_is_a_transpose_layout():
    # out[i][v] = element i%4 of the chunk of lane 4v + i/4: flat source index
    # 4*src + elem = i + 16 v, i.e. the layout (16,4):(1,16) over (i, v).
    pts = [(i, v) for v in range(4) for i in range(16)]
    got = thl.thl_kernel_index_map("tr16_source", pts)
    assert [4 * s + e for s, e in got] == _eval("(16,4):(1,16)", 64)


ROW = 64  # bytes of K staged per operand row (one K-step)


def test_lds_swizzle_is_the_xor_composition():
    # lds_offset(row, b) = Swz<2,4,4>(Swz<2,4,2>(row*64 + b)) over 256 rows.
    rows = 256
    pts = [(r, b) for r in range(rows) for b in range(ROW)]
    got = [o for o, _ in thl.thl_kernel_index_map("lds_offset", pts)]
    linear = f"{rows * ROW}:1"
    first = thl.thl_swizzle_eval(2, 4, 2, linear, range(rows * ROW))
    both = thl.thl_swizzle_eval(2, 4, 4, linear, first)
    assert got == both
    assert sorted(got) == list(range(rows * ROW))


def _banks(offsets, window):
    """4-byte banks touched within a `window`-byte bank window."""
    return [(o % window) // 4 for o in offsets]


def test_swizzle_spreads_a_chunk_over_banks():
    # One logical chunk (16 bytes) read from consecutive rows: any 8 rows
    # cover all 32 banks of a 128-byte window, any 16 rows all 64 banks of a
    # 256-byte window -- no bank is hit twice.
    for chunk in range(ROW // 16):
        for r0 in range(0, 256, 8):
            offs = [thl.thl_kernel_index_map("lds_offset", [(r, chunk * 16 + q)])[0][0]
                    for r in range(r0, r0 + 8) for q in range(0, 16, 4)]
            assert sorted(_banks(offs, 128)) == list(range(32))
        for r0 in range(0, 256, 16):
            offs = [thl.thl_kernel_index_map("lds_offset", [(r, chunk * 16 + q)])[0][0]
                    for r in range(r0, r0 + 16) for q in range(0, 16, 4)]
            assert sorted(_banks(offs, 256)) == list(range(64))


@pytest.mark.parametrize("loadw", [16, 4])
def test_copy_source_inverts_the_lds_layout(loadw):
    # Lane `lane` of the copy instruction at LDS byte `base` writes LDS bytes
    # base + lane*loadw; the (row, byte) it fetches must be stored exactly there.
    rows = 256
    total = rows * ROW
    pts = [(base, lane) for base in range(0, total, 64 * loadw) for lane in range(64)]
    src = thl.thl_kernel_index_map("copy_source", pts, (loadw,))
    back = thl.thl_kernel_index_map("lds_offset", src)
    assert [o for o, _ in back] == [base + lane * loadw for base, lane in pts]
    # one wave instruction covers whole rows, each a contiguous 64-byte run of K
    for base in range(0, total, 64 * loadw):
        got = thl.thl_kernel_index_map("copy_source", [(base, lane) for lane in range(64)], (loadw,))
        rows_hit = {}
        for r, b in got:
            rows_hit.setdefault(r, []).append(b)
        assert len(rows_hit) == max(1, 64 * loadw // ROW)
        for r, bs in rows_hit.items():
            spans = sorted(x for b in bs for x in range(b, b + loadw))
            assert spans == list(range(min(spans), min(spans) + len(spans)))


@pytest.mark.parametrize("count", [8, 64, 1024, 1000])
def test_xcd_remap_is_the_layout(count):
    got = [r for r, _ in thl.thl_kernel_index_map("xcd_remap", [(w, 0) for w in range(count)], (count,))]
    if count % 8 == 0:
        assert got == _eval(f"(8,{count // 8}):({count // 8},1)", count)
    else:
        assert got == list(range(count))
    assert sorted(got) == list(range(count))


@pytest.mark.parametrize("tm,tn,group", [(32, 32, 8), (16, 8, 4), (8, 8, 8), (17, 4, 8), (5, 3, 2)])
def test_grouped_raster_is_the_layout(tm, tn, group):
    count = tm * tn
    got = thl.thl_kernel_index_map("grouped_tile", [(i, 0) for i in range(count)], (tm, tn, group))
    flat = [a + tm * b for a, b in got]
    assert sorted(flat) == list(range(count))  # every tile exactly once
    if tm % group == 0:
        assert flat == _eval(f"({group},{tn},{tm // group}):(1,{tm},{group})", count)
    else:
        full = (tm // group) * group * tn  # whole bands follow the layout
        if full:
            assert flat[:full] == _eval(f"({group},{tn},{tm // group}):(1,{tm},{group})", full)
        rest = tm - (tm // group) * group  # the last band is narrower
        assert flat[full:] == [(tm - rest) + a + tm * b for b in range(tn) for a in range(rest)]


def test_transposed_read_lands_the_mfma_operand_layout():
    # Compose: lane l of group G addresses chunk (k, m) = tr16_operand(l, h);
    # after the transposed read, lane i of the group holds, as value v,
    # element i%4 of the chunk addressed by lane 4v + i/4.  The result must be
    # the 32x32x16 operand map: row l % 32, k = 8*(l/32) + 4h + v.
    for h in (0, 1):
        for l in range(64):
            g, i = l // 16, l % 16
            for v in range(4):
                (src, elem), = thl.thl_kernel_index_map("tr16_source", [(i, v)])
                (k, m), = thl.thl_kernel_index_map("tr16_operand", [(16 * g + src, h)])
                got = (m + elem, k)
                (row, kk), = thl.thl_kernel_index_map("mfma32_operand", [(l, 4 * h + v)], (8,))
                assert got == (row, kk), (h, l, v)


@pytest.mark.parametrize("pitch", [256, 512])
def test_mm_lds_layout_is_a_bijection_and_copy_inverts_it(pitch):
    rows = 32
    pts = [(k, b) for k in range(rows) for b in range(pitch)]
    offs = [o for o, _ in thl.thl_kernel_index_map("mm_lds_offset", pts, (pitch,))]
    assert sorted(offs) == list(range(rows * pitch))
    for loadw in (16, 4):
        src = thl.thl_kernel_index_map(
            "mm_copy_source", [(base, lane) for base in range(0, rows * pitch, 64 * loadw) for lane in range(64)],
            (loadw, pitch))
        back = thl.thl_kernel_index_map("mm_lds_offset", src, (pitch,))
        assert [o for o, _ in back] == [base + lane * loadw for base in range(0, rows * pitch, 64 * loadw)
                                        for lane in range(64)]


@pytest.mark.parametrize("pitch", [256, 512])
def test_transposed_reads_spread_over_banks(pitch):
    # Each 16-lane group reads 16 eight-byte chunks (4 k-rows x 32 bytes):
    # with the k-row swizzle no 4-byte bank of a 256-byte window is hit twice.
    for r0 in (0, 32, 64, 96):
        for ks in (0, 1):
            for h in (0, 1):
                for g in range(4):
                    banks = []
                    for i in range(16):
                        (k, m), = thl.thl_kernel_index_map("tr16_operand", [(16 * g + i, h)])
                        (o, _), = thl.thl_kernel_index_map("mm_lds_offset", [(k + 16 * ks, 2 * (r0 + m))], (pitch,))
                        banks += [(o % 256) // 4, (o % 256) // 4 + 1]
                    assert len(set(banks)) == 32


# ------------------------------------------------------------ paired stages

def test_pair_layout_is_a_bijection_of_two_stages():
    # Stages 2j and 2j+1 of 256 rows x 64 bytes fill one 32 KB pair buffer
    # exactly once between them.
    rows = 256
    offs = []
    for odd in (0, 1):
        pts = [(r, b) for r in range(rows) for b in range(ROW)]
        offs += [o for o, _ in thl.thl_kernel_index_map("pair_lds_offset", pts, (odd,))]
    assert sorted(offs) == list(range(2 * rows * ROW))


def test_pair_rows_keep_the_chunk_swizzle():
    # Inside a row the bytes sit exactly as in a single stage; rows move by
    # whole 512-byte halves of a 1 KB group, so the bank of every byte is
    # unchanged (512 is a multiple of the 256-byte bank window).
    for odd in (0, 1):
        pts = [(r, b) for r in range(0, 256, 3) for b in range(0, ROW, 4)]
        pair = thl.thl_kernel_index_map("pair_lds_offset", pts, (odd,))
        single = thl.thl_kernel_index_map("lds_offset", pts)
        for (po, _), (so, _), (r, _b) in zip(pair, single, pts):
            assert po - so == (r >> 3) * 512 + odd * 512
            assert po % 256 == so % 256


def test_pair_copy_source_inverts_the_pair_layout_with_whole_lines():
    # Lane l of the copy for 1 KB group g writes LDS bytes 1024 g + 16 l ..;
    # the (row, byte of the pair's 128) it fetches must be stored exactly
    # there, and one instruction reads 8 whole 128-byte rows (cache lines).
    for g in range(32):
        got = thl.thl_kernel_index_map("pair_copy_source", [(g, lane) for lane in range(64)])
        back = []
        for r, b in got:
            back.append(thl.thl_kernel_index_map("pair_lds_offset", [(r, b % 64)], (b // 64,))[0][0])
        assert back == [1024 * g + 16 * lane for lane in range(64)]
        rows = {}
        for r, b in got:
            rows.setdefault(r, []).extend(range(b, b + 16))
        assert sorted(rows) == list(range(8 * g, 8 * g + 8))
        assert all(sorted(v) == list(range(128)) for v in rows.values())


def test_pair_copy_lane_part_is_the_same_for_every_group_of_a_wave():
    # A wave copies groups wave, wave + 4, wave + 8, ...: the lane's byte in
    # the pair is the same for all of them (the swizzle repeats every 4
    # groups), so one per-lane offset plus a uniform row step serves all.
    for wave in range(4):
        first = thl.thl_kernel_index_map("pair_copy_source", [(wave, lane) for lane in range(64)])
        for j in range(1, 8):
            g = 4 * j + wave
            got = thl.thl_kernel_index_map("pair_copy_source", [(g, lane) for lane in range(64)])
            assert [(r - 8 * g, b) for r, b in got] == [(r - 8 * wave, b) for r, b in first]
