"""Who may use what (CPU, static checks of the source tree).

The fp64 oracle is test infrastructure: only the tests, the smoke check of the entry script
and the CPU-baseline leg of bench.py may import it, and it imports nothing from the library.
The library and its binding never touch the oracle, so a result that passes parity cannot
have come from it; and no committed file refers to the untracked scratch folder that
.gitignore excludes."""

import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SCRATCH = re.compile(r"\b_work\b")   # the folder name on its own, not inside an identifier


def sources(top, exts=(".py", ".hip", ".h", ".cpp")):
    for dirpath, dirnames, filenames in os.walk(os.path.join(ROOT, top)):
        dirnames[:] = [d for d in dirnames if d not in ("__pycache__", "_build")]
        for f in filenames:
            if f.endswith(exts):
                yield os.path.join(dirpath, f)


def test_oracle_imports_nothing_from_the_library():
    for path in sources("oracle"):
        text = open(path).read()
        assert not re.search(r"^\s*(import|from)\s+online_softmax_07_amd", text, flags=re.M), path
        assert "libfa_mi355x" not in text and "ctypes" not in text, path


def test_library_never_uses_the_oracle():
    for path in sources("online_softmax_07_amd"):
        text = open(path).read()
        assert not re.search(r"^\s*(import|from)\s+oracle", text, flags=re.M), path
        assert "fa_oracle" not in text, path


def test_only_tests_smoke_and_cpu_baseline_import_the_oracle():
    allowed = {os.path.join(ROOT, "bench.py"), os.path.join(ROOT, "__graft_entry__.py")}
    for top in ("online_softmax_07_amd", "include", "profiles"):
        for path in sources(top, exts=(".py", ".hip", ".h", ".cpp", ".txt", ".json")):
            assert "fa_oracle" not in open(path).read(), path
    for path in allowed:
        text = open(path).read()
        uses = [m.start() for m in re.finditer(r"import oracle\.fa_oracle", text)]
        assert len(uses) == 1, (path, len(uses))
    bench = open(os.path.join(ROOT, "bench.py")).read()
    i = bench.index("import oracle.fa_oracle")
    assert "def cpu_baseline" in bench[max(0, i - 2000):i], "bench.py imports the oracle outside cpu_baseline"
    entry = open(os.path.join(ROOT, "__graft_entry__.py")).read()
    i = entry.index("import oracle.fa_oracle")
    assert "def smoke" in entry[max(0, i - 1500):i], "__graft_entry__ imports the oracle outside smoke()"


def test_nothing_committed_reads_the_scratch_folder():
    for top in ("online_softmax_07_amd", "oracle", "tests", "include"):
        for path in sources(top):
            if os.path.abspath(path) == os.path.abspath(__file__):
                continue
            assert not SCRATCH.search(open(path).read()), path
    for f in ("bench.py", "__graft_entry__.py"):
        assert not SCRATCH.search(open(os.path.join(ROOT, f)).read()), f
