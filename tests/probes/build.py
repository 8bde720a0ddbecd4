"""Builds tests/probes/liblayout_probe.so (gfx950 instruction-semantics probes)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "layout_probe.hip")
LIB_PATH = os.path.join(HERE, "liblayout_probe.so")


def _pkg_build_module():
    """The package's build module, loaded by path so that the package itself
    (which loads the HIP library) is not imported."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_vdx_pkg_build", os.path.join(ROOT, "spatiotemporal_attention_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def build_probes(verbose: bool = False) -> str:
    pb = _pkg_build_module()
    HIPCC_FLAGS, hipcc = pb.HIPCC_FLAGS, pb.hipcc
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_probes(verbose=True))
