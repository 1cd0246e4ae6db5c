import importlib.util
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

LIB = ROOT / "vocab_selected_token_amd" / "librlk_logp.so"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct MI355X (gfx950) GPU")
    # a fresh checkout has no built library: build it once (hipcc cross-compiles
    # for gfx950 without a GPU); a built one is used as it is
    if not LIB.exists():
        spec = importlib.util.spec_from_file_location(
            "_rlk_build_lib", ROOT / "vocab_selected_token_amd" / "build_lib.py")
        build_lib = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(build_lib)
        build_lib.build()
    consumer = ROOT / "tests" / "_bin" / "abi_consumer"
    if not consumer.exists():
        import subprocess

        import __graft_entry__

        try:
            __graft_entry__.build_abi_consumer()
        except (OSError, subprocess.CalledProcessError) as exc:
            # only the GPU test of the C consumer needs it; that test reports the absence
            print(f"conftest: C ABI consumer not built: {exc}", file=sys.stderr)
