"""Compile the HIP library in-tree for gfx950: selective_state_space_61_amd/libssm61.so."""
from __future__ import annotations

import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libssm61.so")
SOURCES = [os.path.join(CSRC, f) for f in ("ssm_api.hip", "scan_f32.hip", "scan_bf16.hip", "scan_zoh_f32.hip",
                                            "scan_zoh_bf16.hip", "ssd_bf16.hip", "scan_rows.hip", "scan_time.hip",
                                            "scan_bwd_rows.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("ssm_device.hpp", "scan_fwd.hpp", "scan_table.hpp", "scan_rows.hpp", "scan_rows_table.hpp", "scan_time.hpp", "scan_time_table.hpp", "state_update.hpp",
                                                  "conv1d.hpp", "scan_bwd.hpp", "scan_bwd_rows.hpp", "ssd_fwd.hpp")] + [
    os.path.join(os.path.dirname(HERE), "include", "ssm.h")]
OBJDIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 anywhere (the host pass warns that it does not know
# the feature; that is harmless).
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
         f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
NOISE = "is not a recognized feature for this target"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines() if NOISE not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Always recompiles (the caller asked for a build): one object per source, compiled in
    parallel, then linked into the shared library."""
    from concurrent.futures import ThreadPoolExecutor
    t0 = time.time()
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, os.path.basename(s) + ".o") for s in SOURCES]
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        errs = list(ex.map(lambda so: _run(["hipcc", *FLAGS, "-c", "-o", so[1], so[0]]), zip(SOURCES, objs)))
    errs.append(_run(["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", LIBRARY + ".tmp", *objs]))
    os.replace(LIBRARY + ".tmp", LIBRARY)
    if verbose:
        err = "\n".join(e for e in errs if e.strip())
        if err:
            print(err, file=sys.stderr)
        print(f"built {LIBRARY} in {time.time() - t0:.1f}s")
    return LIBRARY


def is_stale() -> bool:
    if not os.path.exists(LIBRARY):
        return True
    lib_t = os.path.getmtime(LIBRARY)
    return any(os.path.getmtime(s) > lib_t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    build(verbose=True)
