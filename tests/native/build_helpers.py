"""Build the tests' HIP helpers in place (gfx950, hipcc). They are test
code, not part of the library: tests/native/libfp8_convert_check.so."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))


def build(verbose: bool = False) -> list:
    sys.path.insert(0, os.path.join(ROOT, "combine_ep_plan_amd"))
    import _build

    flags = [f for f in _build.FLAGS if f not in ("-I", _build.INCLUDE)]
    out = []
    for name in ("fp8_convert_check",):
        lib = os.path.join(HERE, f"lib{name}.so")
        cmd = [_build.HIPCC] + flags + [os.path.join(HERE, f"{name}.hip"), "-o", lib + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(lib + ".tmp", lib)
        out.append(lib)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
