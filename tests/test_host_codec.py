"""Host side of libsbm against the oracle (CPU only; no GPU calls)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle import codec as OC
from oracle import dictionary as OD
from sub_bit_moe_amd import _native as N
from sub_bit_moe_amd import api, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _fnv1a64_bytes(data: bytes) -> int:
    """FNV-1a 64 from its published definition (offset basis, prime)."""
    h = 0xCBF29CE484222325
    for b in data:
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def _fnv1a64(words):
    return _fnv1a64_bytes(np.asarray(words, np.uint32).astype("<u4").tobytes())


def test_fnv1a64_published_vectors():
    """The checker's FNV-1a 64 against the test vectors of the FNV authors'
    reference suite, so the library's dictionary checksum is pinned to the
    published function and not to a copy of itself."""
    assert _fnv1a64_bytes(b"") == 0xCBF29CE484222325
    assert _fnv1a64_bytes(b"a") == 0xAF63DC4C8601EC8C
    assert _fnv1a64_bytes(b"foobar") == 0x85944171F73967E8


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "sbm.h")).read()
    declared = set(re.findall(r"\b(sbm_[a-z0-9_]+)\s*\(", header))
    assert declared, "no declarations found"
    L = N.lib()
    missing = [s for s in declared if not hasattr(L, s)]
    assert not missing, missing
    assert declared == set(N.exported_symbols())


def test_dictionary_bit_exact_with_oracle(odict):
    words, cs = api.build_dictionary(0.885)
    assert np.array_equal(words, odict["words"])
    assert cs == api.dictionary_checksum(words)
    w2, _ = api.build_dictionary(0.886)
    assert np.array_equal(w2, words)


@pytest.mark.parametrize("p0", [0.7, 0.857, 0.95])
def test_dictionary_other_p0_matches_oracle(p0):
    words, _ = api.build_dictionary(p0)
    ref = OD.dictionary_words(OD.build_dictionary(p0))
    assert np.array_equal(words, ref)


def test_dictionary_mismatch_bits():
    """Bits per weight of the greedy encoding of seeded P(0)=0.857 symbols with
    the page's table (p0 = 0.885) and with a table built for the data
    (p0 = 0.857): the matched table spends fewer bits, through entries with a
    fourth nonzero that the page's table does not hold."""
    sym = synth.ternary_symbols(np.random.default_rng(11), 128, 2048, 0.857)
    bits = {}
    for key, p0 in {"static": 0.885, "matched": 0.857}.items():
        w, _ = api.build_dictionary(p0)
        codes, _, _ = api.encode_matrix(sym, w)
        bits[key] = 16.0 * len(codes) / sym.size
        sym28, _ = OD.expansion_table(w)
        bits[key + "_entries_4nz"] = int(((sym28 != 0).sum(axis=1) >= 4).sum())
    assert bits["static"] / bits["matched"] > 1.01, bits
    assert bits["static_entries_4nz"] == 0 and bits["matched_entries_4nz"] > 0, bits


def test_checksum_is_fnv1a64(odict):
    assert api.dictionary_checksum(odict["words"]) == _fnv1a64(odict["words"])


@pytest.mark.parametrize("rows,cols,p0,seed", [(1, 2, 0.886, 1), (17, 30, 0.886, 2), (64, 256, 0.857, 3),
                                               (40, 2080, 0.886, 4), (9, 6144, 0.886, 5),
                                               (31, 98, 0.5, 6), (5, 64, 0.0, 7), (6, 3072, 1.0, 8)])
def test_encoder_bit_exact_with_oracle(odict, rows, cols, p0, seed):
    sym = synth.ternary_symbols(np.random.default_rng(seed), rows, cols, p0)
    codes, row_off, bstart = api.encode_matrix(sym, odict["words"])
    rc, ro = OC.encode_matrix(sym, odict["child"])
    assert np.array_equal(codes, rc)
    assert np.array_equal(row_off, ro)
    assert np.array_equal(bstart, OC.block_starts(rc, odict["lens"], N.SBM_BLOCK))
    api.validate_stream(codes, row_off, rows, cols, odict["words"])
    assert np.array_equal(api.block_starts(codes, odict["words"]), bstart)


def test_encoder_error_paths(odict):
    w = odict["words"]
    with pytest.raises(N.SbmError) as e:
        api.encode_matrix(np.zeros((2, 7), np.uint8), w)
    assert e.value.status == -2
    bad = np.zeros((2, 8), np.uint8)
    bad[1, 3] = 3
    with pytest.raises(N.SbmError) as e:
        api.encode_matrix(bad, w)
    assert e.value.status == -1
    # capacity too small
    sym = np.full((1, 8), 2, np.uint8)
    codes = np.zeros(1, np.uint16)
    row_off = np.zeros(2, np.uint32)
    n = C.c_uint64()
    st = N.lib().sbm_encode_matrix(sym.ctypes.data, 1, 8, w.ctypes.data, codes.ctypes.data, 1,
                                   row_off.ctypes.data, None, C.addressof(n))
    assert st == -6 and n.value == 4
    # a dictionary that is not prefix-closed
    w2 = w.copy()
    c = next(i for i, s in enumerate(odict["seqs"]) if len(s) == 4)
    w2[2 * c] = w2[2 * c + 1] = 0
    with pytest.raises(N.SbmError):
        api.encode_matrix(np.zeros((1, 4), np.uint8), w2)


def test_validate_stream_detects_corruption(odict):
    w = odict["words"]
    sym = synth.ternary_symbols(np.random.default_rng(9), 8, 120, 0.886)
    codes, row_off, _ = api.encode_matrix(sym, w)
    api.validate_stream(codes, row_off, 8, 120, w)
    bad = row_off.copy()
    bad[3] += 1
    with pytest.raises(N.SbmError) as e:
        api.validate_stream(codes, bad, 8, 120, w)
    assert e.value.status == -3
    with pytest.raises(N.SbmError):
        api.validate_stream(codes[:-1], row_off, 8, 120, w)
    trunc = row_off.copy()
    trunc[-1] -= 1
    with pytest.raises(N.SbmError):
        api.validate_stream(codes[:-1], trunc, 8, 120, w)


def _image_fields(img):
    hdr = np.frombuffer(img[:32].tobytes(), np.uint32)
    tab = np.frombuffer(img[32:].tobytes(), np.uint32)
    return int(hdr[1]), int(hdr[2]), int(hdr[3]), tab


def test_decode_image_reproduces_every_codeword(odict):
    """Apply the fused kernel's table arithmetic to all 65536 codewords on the
    CPU and compare run length, nonzero positions and signs with the oracle."""
    img = api.dict_image(odict["words"])
    assert img.size == N.lib().sbm_dict_image_bytes()
    version, H, n_tab, tab = _image_fields(img)
    assert version == 5
    assert n_tab == H + (65536 - H + 7) // 8 and n_tab <= tab.size
    # every codeword from the split on has 3 nonzeros, and the one before not
    nnz = (odict["sym28"] != 0).sum(axis=1)
    assert (nnz[H:] == 3).all() and nnz[H - 1] < 3
    c = np.arange(65536, dtype=np.uint32)
    e = c + np.uint32(7 * H)
    idx = np.minimum(c, e >> np.uint32(3))
    assert idx.max() < n_tab
    assert np.array_equal(idx[H:], H + (c[H:] - H) // 8) and np.array_equal(idx[:H], c[:H])
    slots = tab[idx] + ((e & np.uint32(7)) * np.uint32(0x8102) & np.uint32(0x20202))
    L = (slots >> np.uint32(24)).astype(np.int64)
    assert (L % 6 == 0).all()
    assert np.array_equal(L // 6, odict["lens"])
    sym28 = odict["sym28"]
    for cw in range(65536):
        exp = np.zeros(28, np.uint8)
        for i in range(3):
            byte = (int(slots[cw]) >> (8 * i)) & 0xFF
            if byte == 4:
                continue                       # zero slot
            pos, kk = divmod(byte, 6)
            exp[pos] = 1 if kk == 0 else 2     # triple layout [-x, +x, 0]
        assert np.array_equal(exp, sym28[cw]), cw


def test_image_rejects_non_canonical(odict):
    w = odict["words"].copy()
    # swap two entries of different classes
    w[[2 * 100, 2 * 100 + 1, 2 * 60000, 2 * 60000 + 1]] = w[[2 * 60000, 2 * 60000 + 1, 2 * 100, 2 * 100 + 1]]
    with pytest.raises(N.SbmError) as e:
        api.dict_image(w)
    assert e.value.status == -4
    w3, _ = api.build_dictionary(0.5)         # entries with more than 3 nonzeros
    with pytest.raises(N.SbmError) as e:
        api.dict_image(w3)
    assert e.value.status == -4


@pytest.mark.parametrize("p0", [0.857, 0.864, 0.885])
def test_decode_image4_reproduces_every_codeword(odict_for, p0):
    """The 4-slot image of a table built for P(0) = p0: the fused kernel's
    arithmetic (idx = min(c, (c + 7H) >> 3), word = tab[idx] + spread of the
    sign bits (c + 7H) & 7 into fields 0..2) applied to all 65536 codewords on
    the CPU; 7-bit fields k = 3p + [positive] (2: empty) and L / 2 in bits 28..31
    compared with the oracle's unpacking of the same table."""
    od = odict_for(p0)
    w, _ = api.build_dictionary(p0)
    assert np.array_equal(w, od["words"])
    img = api.dict_image(w, 4)
    assert img.size == N.lib().sbm_dict_image4_bytes()
    version, H, n_tab, tab = _image_fields(img)
    assert version == 6
    assert n_tab == H + (65536 - H + 7) // 8 and n_tab <= tab.size
    nnz = (od["sym28"] != 0).sum(axis=1)
    assert nnz.max() <= 4 and (nnz[H:] >= 3).all()
    c = np.arange(65536, dtype=np.uint32)
    e = c + np.uint32(7 * H)
    idx = np.minimum(c, e >> np.uint32(3))
    assert idx.max() < n_tab
    word = tab[idx] + ((e & np.uint32(7)) * np.uint32(0x1041) & np.uint32(0x4081))
    assert np.array_equal((word >> np.uint32(28)).astype(np.int64) * 2, od["lens"])
    exp = np.zeros((65536, 28), np.uint8)
    filled = np.zeros(65536, np.int64)
    for i in range(4):
        k = ((word >> np.uint32(7 * i)) & np.uint32(0x7F)).astype(np.int64)
        live = k != 2
        assert (k[live] % 3 != 2).all()                  # only the empty slot reads a zero
        pos, sgn = k // 3, k % 3
        assert (pos[live] < od["lens"][live]).all()
        exp[c[live], pos[live]] = (1 + sgn[live]).astype(np.uint8)
        filled += live
    assert np.array_equal(filled, nnz)
    assert np.array_equal(exp, od["sym28"])
    if p0 == 0.857:
        assert H == 9734 and n_tab == 16710 and (nnz == 4).sum() == 1376


def test_image4_rejections(odict):
    w = odict["words"].copy()
    w[[2 * 100, 2 * 100 + 1, 2 * 60000, 2 * 60000 + 1]] = w[[2 * 60000, 2 * 60000 + 1, 2 * 100, 2 * 100 + 1]]
    with pytest.raises(N.SbmError) as e:
        api.dict_image(w, 4)
    assert e.value.status == -4
    for p0 in (0.5, 0.8, 0.856):      # more than 4 nonzeros; 31634 and 18250 table words
        with pytest.raises(N.SbmError) as e:
            api.dict_image(api.build_dictionary(p0)[0], 4)
        assert e.value.status == -4
    w857, _ = api.build_dictionary(0.857)
    with pytest.raises(N.SbmError) as e:
        api.dict_image(w857)                   # the 3-slot image cannot hold it
    assert e.value.status == -4
    with pytest.raises(N.SbmError) as e:
        N.check(N.lib().sbm_dict_image4(w857.ctypes.data, np.zeros(64, np.uint8).ctypes.data, 64))
    assert e.value.status == -6


def _div_magic(d):
    l = 0
    while (1 << l) < d:
        l += 1
    return (1 << (30 + l)) // d + 1, 30 + l


@pytest.mark.parametrize("cols", [2, 6, 30, 256, 768, 2080, 3072, 6144, 13000])
def test_division_magic_exact(cols):
    """Granlund-Montgomery exact division used by the kernel for numerators
    below 2^30 (positions in 6-byte units)."""
    d = 6 * cols
    m, s = _div_magic(d)
    rng = np.random.default_rng(cols)
    n = np.concatenate([rng.integers(0, 1 << 30, 20000), np.arange(0, 5 * d), [(1 << 30) - 1]])
    n = n.astype(object)
    assert all((int(v) * m) >> s == int(v) // d for v in n[::7])


def test_fused_argument_errors_without_gpu():
    L = N.lib()
    z = None
    # odd width, bad flags, bad shape are rejected before any device call
    assert L.sbm_moe_fused_decode_matvec(z, z, z, z, z, 1, 4, 7, z, z, z, 1, z, 0, z, 0, z) == -2
    assert L.sbm_moe_fused_decode_matvec(z, z, z, z, z, 1, 4, 8, z, z, z, 1, z, 256, z, 0, z) == -1
    assert L.sbm_moe_fused_decode_matvec(z, z, z, z, z, 1, 4, 8, z, z, z, 1, z, 64 | 8, z, 0, z) == -1
    assert L.sbm_moe_fused_decode_matvec(z, z, z, z, z, 1, 4, 8, z, z, z, 1, z, 128 | 8, z, 0, z) == -1
    assert L.sbm_moe_fused_decode_matvec(z, z, z, z, z, 1, 4, 8, z, z, z, 1, z, 128, z, 0, z) == -1   # null pointers
    assert L.sbm_moe_fused_decode_matvec(z, z, z, z, z, 1, 4, 8, z, z, z, 1, z, 64, z, 0, z) == -1   # null pointers
    assert L.sbm_moe_fused_decode_matvec(z, z, z, z, z, 1, 4, 8, z, z, z, 1, z, 16 | 8, z, 0, z) == -1
    assert L.sbm_moe_fused_decode_matvec(z, z, z, z, z, 1, 4, 8, z, z, z, 1, z, 32 | 8, z, 0, z) == -1
    assert L.sbm_moe_fused_decode_matvec(z, z, z, z, z, 0, 4, 8, z, z, z, 1, z, 0, z, 0, z) == -1
    assert L.sbm_moe_fused_decode_matvec(z, z, z, z, z, 1, 4, 8, z, z, z, 0, z, 0, z, 0, z) == 0
    assert L.sbm_moe_fused_decode_matvec(z, z, z, z, z, 1, 4, 8, z, z, z, 3, z, 0, z, 0, z) == -1
    assert L.sbm_moe_fused_decode_matvec(z, z, z, z, z, 1, 1 << 23, 6144, z, z, z, 1, z, 0, z, 0, z) == -5
    assert L.sbm_decode_ref(z, z, 3, 5, z, z, z, z) == -2
    assert L.sbm_decode_dense(z, 10, z, 3, 5, z, 0, z, z, z) == -2          # odd width
    assert L.sbm_decode_dense(z, 0, z, 0, 4, z, 0, z, z, z) == 0            # no rows: nothing to do
    assert L.sbm_decode_dense(z, 0, z, 3, 4, z, 0, z, z, z) == -1           # rows without codewords
    assert L.sbm_decode_dense(z, 10, z, 1 << 20, 1 << 12, z, 0, z, z, z) == -5   # positions beyond 32 bits
    assert L.sbm_decode_dense(z, 10, z, 3, 4, z, 0, z, z, z) == -1          # null pointers
    assert L.sbm_decode_ref(z, z, 0, 4, z, z, z, z) == 0
    assert L.sbm_workspace_bytes(10, 5) >= 4 * (16 + 10 + 11 + 11 + 5)


@pytest.mark.parametrize("E,rows,cols,p0,dict_p0", [(5, 70, 514, 0.886, 0.885), (1, 1, 2, 0.886, 0.885),
                                                    (3, 300, 2080, 0.857, 0.857), (2, 0, 30, 0.886, 0.885)])
def test_encode_experts_layout(odict_for, E, rows, cols, p0, dict_p0):
    """The native whole-projection encoder against per-matrix encodes
    assembled by the binding: same aligned code bases, padding, offsets, block
    starts and descriptors; the first matrix's codes bit-exact with the
    oracle's encoder."""
    od = odict_for(dict_p0)
    w = od["words"]
    rng = np.random.default_rng(rows + E)
    syms = [synth.ternary_symbols(rng, rows, cols, p0) for _ in range(E)]
    scs = [synth.row_scales(rng, rows) for _ in range(E)]
    codes, row_off, bstart, descs = api.encode_experts(syms, w)
    tag = api.dict_tag(w)
    ref = api.ExpertStack.assemble([api.encode_matrix(s, w) + (sc,) for s, sc in zip(syms, scs)], rows, cols, tag)
    assert np.array_equal(codes, ref[1]) and np.array_equal(row_off, ref[2]) and np.array_equal(bstart, ref[3])
    assert [bytes(a) for a in descs] == [bytes(b) for b in ref[0]]
    # every descriptor names its dictionary: the low half of the FNV-1a 64 checksum of the packed table
    assert all(d.dict_tag == (_fnv1a64(w) & 0xFFFFFFFF) for d in descs)
    assert all(d.code_base % N.SBM_CODE_ALIGN == 0 for d in descs)
    if rows:
        rc, ro = OC.encode_matrix(syms[0], od["child"])
        d = descs[0]
        assert np.array_equal(codes[d.code_base:d.code_base + d.n_codes], rc)
        assert np.array_equal(row_off[:rows + 1], ro)


def test_encode_experts_errors(odict):
    w = odict["words"]
    L = N.lib()
    bad = np.zeros((2, 8), np.uint8)
    bad[1, 3] = 3
    odd = np.zeros((2, 7), np.uint8)
    nc, nb = C.c_uint64(), C.c_uint64()
    for m, status in ((bad, -1), (odd, -2)):
        ptrs = (C.c_void_p * 1)(m.ctypes.data)
        assert L.sbm_encode_experts(1, ptrs, m.shape[0], m.shape[1], w.ctypes.data, None, 0, None, None, 0, None,
                                    C.addressof(nc), C.addressof(nb)) == status
    good = np.full((3, 64), 2, np.uint8)                  # all nonzero: 32 codewords per row
    ptrs = (C.c_void_p * 2)(good.ctypes.data, good.ctypes.data)
    assert L.sbm_encode_experts(2, ptrs, 3, 64, w.ctypes.data, None, 0, None, None, 0, None,
                                C.addressof(nc), C.addressof(nb)) == -6
    assert nc.value == 2 * 96 and nb.value == 2      # 96 per matrix, already a multiple of 8
    with pytest.raises(ValueError):
        api.encode_experts([good, np.zeros((3, 62), np.uint8)], w)
