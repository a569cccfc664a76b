"""The hot path driven from plain C on the GPU, with no PyTorch in the process:
tests/c/fc1_from_c.c runs three delayed-scaling steps of a small FC1-shaped
layer (fp8_quantize_update of X and of W with its transposed codes, then the
exact fp8_gemm) through include/fp8mi.h and the HIP runtime's C API, and writes
every input and output.  Here the CPU oracle replays the same steps:
codes, amax, scales, history, head and status bit for bit
("4.2 Hopper I — Transformer Engine·FP8", §4.2.4 amax and scale, §4.2.6 the
recipe: history of 16, max rule), the GEMM within 1e-5·Σ|ab| (§4.2.4 FP32
accumulation and the ×1/scale restore)."""

import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import fp8_precision_numerics_amd as fm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from oracle import gemm as ogemm  # noqa: E402
from oracle import scaling  # noqa: E402

M, K, N, L, STEPS = 256, 512, 384, 16, 3


def _state(path):
    raw = open(path, "rb").read()
    f = np.frombuffer(raw[:16], dtype=np.float32)
    i = np.frombuffer(raw[16:24], dtype=np.int32)
    h = np.frombuffer(raw[24:], dtype=np.float32)
    return {"amax": f[0], "scale": f[1], "scale_inv": f[2], "scale_inv_used": f[3], "head": int(i[0]),
            "status": int(i[1]), "history": h}


def _bits(v):
    return np.asarray(v, dtype=np.float32).view(np.uint32)


@pytest.mark.gpu
@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_fc1_steps_from_plain_c(tmp_path):
    lib = fm.load_library()
    libdir = os.path.dirname(lib._name)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = tmp_path / "fc1_from_c"
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "fc1_from_c.c"), "-L", libdir, "-lfp8mi",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", f"-Wl,-rpath,{libdir}",
           f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = tmp_path / "out"
    out.mkdir()
    print(f"running {exe} (M={M} K={K} N={N}, {STEPS} steps)", flush=True)
    run = subprocess.run([str(exe), str(out)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr

    st = {"x": scaling.DelayedScaling("e4m3", L), "w": scaling.DelayedScaling("e4m3", L)}
    for t in range(STEPS):
        x = np.fromfile(out / f"x{t}.bin", dtype=np.uint16).reshape(M, K)
        w = np.fromfile(out / f"w{t}.bin", dtype=np.uint16).reshape(K, N)
        qx = np.fromfile(out / f"qx{t}.bin", dtype=np.uint8).reshape(M, K)
        qwt = np.fromfile(out / f"qwt{t}.bin", dtype=np.uint8).reshape(N, K)
        c = np.fromfile(out / f"c{t}.bin", dtype=np.float32).reshape(M, N)
        used = {}
        for name, data, codes in (("x", x, qx), ("w", w, qwt.T)):
            ref = st[name]
            used[name] = ref.scale_inv
            want, amax, _ = scaling.quantize(scaling.widen(data, "bf16"), ref.scale, "e4m3")
            assert np.array_equal(codes, want), (t, name, int(np.count_nonzero(codes != want)))
            ref.update(amax)
            got = _state(out / f"s{name}{t}.bin")
            assert _bits(got["amax"]) == _bits(amax), (t, name)
            assert _bits(got["scale"]) == _bits(ref.scale), (t, name, got["scale"], ref.scale)
            assert _bits(got["scale_inv"]) == _bits(ref.scale_inv), (t, name)
            assert _bits(got["scale_inv_used"]) == _bits(used[name]), (t, name)
            assert got["head"] == ref.head and got["status"] == ref.status, (t, name)
            assert np.array_equal(_bits(got["history"]), _bits(ref.history)), (t, name)
        want_c = ogemm.dequant_gemm(qx, "e4m3", qwt.T, "e4m3", used["x"], used["w"])
        bound = ogemm.abs_bound(qx, "e4m3", qwt.T, "e4m3", used["x"], used["w"])
        err = np.abs(c.astype(np.float64) - want_c)
        assert np.all(err <= bound), (t, float((err - bound).max()))
    # the activations grew every step: the delayed scale trails them
    assert st["x"].scale < np.float32(448.0) / np.float32(2.0)
