import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (HIP device)")


@pytest.fixture(scope="session")
def odict():
    """The oracle's default dictionary (p0 = 0.885) with derived helpers."""
    from oracle import dictionary as D
    from oracle import codec as C
    seqs = D.build_dictionary(0.885)
    words = D.dictionary_words(seqs)
    sym28, lens = D.expansion_table(words)
    child = C.trie_children(seqs)
    return {"seqs": seqs, "words": words, "sym28": sym28, "lens": lens, "child": child}


_ODICTS = {}


@pytest.fixture(scope="session")
def odict_for(odict):
    """The oracle's dictionary for another p0 (cached), same fields as odict."""
    from oracle import dictionary as D
    from oracle import codec as C

    def make(p0):
        if p0 == 0.885:
            return odict
        if p0 not in _ODICTS:
            seqs = D.build_dictionary(p0)
            words = D.dictionary_words(seqs)
            sym28, lens = D.expansion_table(words)
            _ODICTS[p0] = {"seqs": seqs, "words": words, "sym28": sym28, "lens": lens,
                           "child": C.trie_children(seqs)}
        return _ODICTS[p0]
    return make
