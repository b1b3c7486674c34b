"""The product path has no fallback and shares no code with the oracle: the
package never imports the oracle, the oracle imports nothing but numpy and
the standard library, and with its HIP library missing every call fails
loudly instead of computing anything on the CPU (no GPU needed)."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "decode_kv_cache_evict_amd")


def test_package_sources_do_not_reference_the_oracle():
    for name in sorted(os.listdir(PKG)):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(PKG, name)).read())
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                assert not any(a.name.split(".")[0] == "oracle" for a in node.names), name
            if isinstance(node, ast.ImportFrom):
                assert (node.module or "").split(".")[0] != "oracle", name


def test_oracle_does_not_reference_the_package():
    odir = os.path.join(ROOT, "oracle")
    for name in sorted(os.listdir(odir)):
        if not name.endswith(".py"):
            continue
        src = open(os.path.join(odir, name)).read()
        tree = ast.parse(src)
        mods = [a.name for n in ast.walk(tree) if isinstance(n, ast.Import) for a in n.names]
        mods += [n.module or "" for n in ast.walk(tree) if isinstance(n, ast.ImportFrom)]
        assert all(m.split(".")[0] in ("math", "numpy", "oracle", "") or m.startswith("kvevict_oracle")
                   for m in mods), (name, mods)
        assert "decode_kv_cache_evict_amd" not in src and "csrc" not in src, name


def test_missing_library_raises():
    code = (
        "import decode_kv_cache_evict_amd as kv\n"
        "try:\n"
        "    kv.lib()\n"
        "except RuntimeError as e:\n"
        "    assert 'missing' in str(e), e\n"
        "    print('raised')\n"
        "else:\n"
        "    raise SystemExit('loaded without a library')\n"
        "import sys\n"
        "assert 'oracle' not in sys.modules\n"
    )
    env = dict(os.environ, KVE_LIB=os.path.join(ROOT, "no_such_dir", "libkvevict.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "raised" in r.stdout, r.stderr[-2000:]
