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
