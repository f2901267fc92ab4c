"""The host codec (dictionary, decode images, trie encoder, block starts,
stream validation: sbm_host.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer by g++ and driven through the C ABI in a child
process (the sanitizer runtime must be loaded first), on seeded inputs,
edge shapes and error paths.  Every result is compared with the regular
library's, which the other CPU tests pin to the oracle; any sanitizer report
fails the child."""
import json
import os
import shutil
import subprocess
import sys
import textwrap

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build", "sanitized")

CHILD = textwrap.dedent(r'''
    import ctypes as C, json, sys
    import numpy as np
    lib = C.CDLL(sys.argv[1])
    P = C.c_void_p
    lib.sbm_build_dictionary.argtypes = [C.c_double, P, P]
    lib.sbm_dict_image.argtypes = [P, P, C.c_size_t]
    lib.sbm_dict_image4.argtypes = [P, P, C.c_size_t]
    lib.sbm_dict_image_bytes.restype = C.c_size_t
    lib.sbm_dict_image4_bytes.restype = C.c_size_t
    lib.sbm_encode_size.argtypes = [P, C.c_int32, C.c_int32, P, P]
    lib.sbm_encode_matrix.argtypes = [P, C.c_int32, C.c_int32, P, P, C.c_uint64, P, P, P]
    lib.sbm_encode_experts.argtypes = [C.c_int32, P, C.c_int32, C.c_int32, P, P, C.c_uint64, P, P, C.c_uint64,
                                       P, P, P]
    lib.sbm_validate_stream.argtypes = [P, C.c_uint64, P, C.c_int32, C.c_int32, P]
    lib.sbm_block_starts.argtypes = [P, C.c_uint64, P, P]
    lib.sbm_build_trie.argtypes = [P, P]
    lib.sbm_trie_words.restype = C.c_size_t
    out = {}
    rng = np.random.default_rng(5)
    for p0 in (0.885, 0.857):
        w = np.zeros(131072, np.uint32); cs = C.c_uint64()
        assert lib.sbm_build_dictionary(p0, w.ctypes.data, C.addressof(cs)) == 0
        out[f"dict_{p0}"] = int(w.astype(np.uint64).sum()), cs.value
        n = lib.sbm_dict_image4_bytes() if p0 < 0.885 else lib.sbm_dict_image_bytes()
        im = np.zeros(n, np.uint8)
        f = lib.sbm_dict_image4 if p0 < 0.885 else lib.sbm_dict_image
        assert f(w.ctypes.data, im.ctypes.data, n) == 0
        out[f"image_{p0}"] = int(im.astype(np.uint64).sum())
        trie = np.zeros(lib.sbm_trie_words(), np.int32)
        assert lib.sbm_build_trie(w.ctypes.data, trie.ctypes.data) == 0
        out[f"trie_{p0}"] = int(trie.astype(np.int64).sum())
        for rows, cols, q in ((1, 2, 0.5), (3, 30, 0.886), (37, 514, p0), (64, 2080, 0.886), (5, 98, 0.0), (4, 60, 1.0)):
            u = rng.random((rows, cols))
            sym = np.where(u < q, 0, np.where(rng.random((rows, cols)) < 0.5, 1, 2)).astype(np.uint8)
            nn = C.c_uint64()
            assert lib.sbm_encode_size(sym.ctypes.data, rows, cols, w.ctypes.data, C.addressof(nn)) == 0
            codes = np.zeros(max(nn.value, 1), np.uint16); roff = np.zeros(rows + 1, np.uint32)
            bst = np.zeros(max((nn.value + 1023) // 1024, 1), np.uint32)
            assert lib.sbm_encode_matrix(sym.ctypes.data, rows, cols, w.ctypes.data, codes.ctypes.data, codes.size,
                                         roff.ctypes.data, bst.ctypes.data, C.addressof(nn)) == 0
            assert lib.sbm_validate_stream(codes.ctypes.data, nn.value, roff.ctypes.data, rows, cols, w.ctypes.data) == 0
            b2 = np.zeros_like(bst)
            assert lib.sbm_block_starts(codes.ctypes.data, nn.value, w.ctypes.data, b2.ctypes.data) == 0
            assert np.array_equal(b2, bst)
            key = f"enc_{p0}_{rows}x{cols}"
            out[key] = [int(nn.value), int(codes[:nn.value].astype(np.int64).sum()), roff.tolist()[-1]]
            if nn.value > 1:                      # damaged streams are refused, never read out of bounds
                bad = codes.copy(); bad[nn.value // 2] = 65535
                out[key + "_bad"] = lib.sbm_validate_stream(bad.ctypes.data, nn.value, roff.ctypes.data, rows, cols,
                                                            w.ctypes.data)
                roff2 = roff.copy(); roff2[-1] += 3
                out[key + "_badoff"] = lib.sbm_validate_stream(codes.ctypes.data, nn.value, roff2.ctypes.data, rows,
                                                               cols, w.ctypes.data)
        mats = [np.where(rng.random((9, 770)) < 0.886, 0, 1 + (rng.random((9, 770)) < 0.5)).astype(np.uint8)
                for _ in range(3)]
        ptrs = (C.c_void_p * 3)(*[m.ctypes.data for m in mats])
        nc, nb = C.c_uint64(), C.c_uint64()
        assert lib.sbm_encode_experts(3, ptrs, 9, 770, w.ctypes.data, None, 0, None, None, 0, None,
                                      C.addressof(nc), C.addressof(nb)) == -6
        codes = np.zeros(nc.value, np.uint16); roff = np.zeros(3 * 10, np.uint32); bst = np.zeros(nb.value, np.uint32)
        desc = (C.c_uint8 * (48 * 3))()
        assert lib.sbm_encode_experts(3, ptrs, 9, 770, w.ctypes.data, codes.ctypes.data, codes.size, roff.ctypes.data,
                                      bst.ctypes.data, bst.size, desc, C.addressof(nc), C.addressof(nb)) == 0
        out[f"experts_{p0}"] = [int(codes.astype(np.int64).sum()), roff.tolist(), bst.tolist(), bytes(desc).hex()]
    # error paths: null pointers, odd widths, bad symbols, a table that is not canonical
    z = None
    out["errors"] = [lib.sbm_encode_size(z, 2, 4, z, z), lib.sbm_encode_size(np.zeros(8, np.uint8).ctypes.data, 2, 3,
                     w.ctypes.data, C.addressof(nn)), lib.sbm_validate_stream(z, 0, z, 1, 2, z)]
    w_bad = w.copy(); w_bad[2], w_bad[4] = w_bad[4], w_bad[2]
    im = np.zeros(lib.sbm_dict_image_bytes(), np.uint8)
    out["bad_table_image"] = lib.sbm_dict_image(w_bad.ctypes.data, im.ctypes.data, im.size)
    print(json.dumps(out))
''')


def _build_sanitized():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    os.makedirs(BUILD, exist_ok=True)
    out = os.path.join(BUILD, "libsbm_host_sanitized.so")
    src = os.path.join(ROOT, "sub_bit_moe_amd", "csrc", "sbm_host.cpp")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fPIC", "-shared", f"-I{os.path.join(ROOT, 'include')}",
           f"-I{os.path.join(ROOT, 'sub_bit_moe_amd', 'csrc')}", src, "-o", out, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return gxx, out


def test_host_codec_under_sanitizers():
    gxx, so = _build_sanitized()
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    ubsan = subprocess.run([gxx, "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", CHILD, so], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"sanitized child failed ({r.returncode}):\n{r.stderr[-4000:]}"
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    got = json.loads(r.stdout.strip().splitlines()[-1])
    # the same calls through the regular library
    env2 = dict(os.environ, PYTHONPATH=ROOT)
    from sub_bit_moe_amd import _native as N
    r2 = subprocess.run([sys.executable, "-c", CHILD, N.LIB_PATH], capture_output=True, text=True, env=env2,
                        timeout=600)
    assert r2.returncode == 0, r2.stderr[-4000:]
    ref = json.loads(r2.stdout.strip().splitlines()[-1])
    assert got == ref
    assert ref["bad_table_image"] != 0 and all(e != 0 for e in ref["errors"])
