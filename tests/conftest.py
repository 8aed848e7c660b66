import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_sessionstart(session):
    # The libraries are build products kept out of version control: build
    # them in-tree if this checkout has none yet (hipcc cross-compiles for
    # gfx950 without a GPU).
    pkg = os.path.join(ROOT, "paged_kv_gqa_block_amd")
    if not all(os.path.exists(os.path.join(pkg, n)) for n in ("libpkv.so", "libpkv_probe.so")):
        from paged_kv_gqa_block_amd import build as _build

        _build.build(verbose=True)
