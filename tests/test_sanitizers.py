"""The C test infrastructure (the fp64 oracle, the seeded input generator) under AddressSanitizer
and UndefinedBehaviorSanitizer, on the CPU.

"FlashAttention forward in C" (section 4) runs its test suite under ASan, UBSan and TSan, and its
pitfalls (section 5) include a null pointer plus a zero offset at Tk = 0, which UBSan reports.
Here both C sources are built with gcc -fsanitize=address,undefined (every report fatal), and the
oracle's pins plus the degenerate calls below (Tk = 0, no rows, rows that see nothing, a row
subset, bf16 inputs, masks, sinks, windows, softcap and ALiBi) run against those builds in a
child process with the ASan runtime preloaded.  Only the oracle and the generator run there: the
GPU library is not loaded.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

DEGENERATE = r'''
import sys
import numpy as np
sys.path.insert(0, ROOT)
import oracle, synth
q = synth.normal(synth.seed_of("san", "q"), (2, 4, 9, 8), "f32")
k = synth.normal(synth.seed_of("san", "k"), (2, 2, 11, 8), "f32")
v = synth.normal(synth.seed_of("san", "v"), (2, 2, 11, 8), "f32")
z = synth.normal_f32(synth.seed_of("san", "z"), (4,))
e = np.zeros((2, 2, 0, 8), np.float32)
o, l = oracle.attention(q, e, e, scale=0.3)                          # Tk = 0
assert np.all(o == 0) and np.all(l == -np.inf)
o, l = oracle.attention(q, e, e, scale=0.3, sinks=z)                 # Tk = 0 with sinks
assert np.all(o == 0) and np.allclose(l, np.broadcast_to(z[None, :, None], l.shape))
o, l = oracle.attention(q[:, :, :0], k, v, scale=0.3)                # no rows
assert o.size == 0 and l.size == 0
o, l = oracle.attention(q, k, v, scale=0.3, q_offset=0, causal=True, window=1, rows=np.zeros((0, 3), np.int64))
o, l = oracle.attention(q, k, v, scale=0.3, q_offset=20, causal=True, window=3)   # rows past Tk see the last keys
m = synth.neg_inf_mask(synth.seed_of("san", "m"), (9, 11), 0.4)
m[3] = -np.inf
o, l = oracle.attention(q, k, v, scale=0.3, causal=False, mask=m[None, None], sinks=z)
o, l = oracle.attention(q, k, v, scale=0.3, causal=False, mask=m[None, None])
assert np.all(o[:, :, 3] == 0) and np.all(l[:, :, 3] == -np.inf)
rows = np.array([[0, 0, 0], [1, 3, 8], [1, 0, 4]], np.int64)
o, l = oracle.attention(q, k, v, scale=0.3, causal=True, rows=rows, softcap=5.0, alibi=np.abs(z))
qb, kb, vb = (synth.to_bf16_bits(a) for a in (q, k, v))
o, l = oracle.attention(qb, kb, vb, scale=0.3, causal=True, window=4, sinks=z)
u = synth.uniform(synth.seed_of("san", "u"), (17,), start=5)
assert np.all((u >= 0) & (u < 1))
print("DEGENERATE_OK", flush=True)
'''


def _build(tmp, src, out):
    cmd = ["gcc", *SAN, "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not asan or not os.path.exists(asan):
        pytest.skip("gcc's ASan runtime is not installed")
    orc = _build(tmp_path, os.path.join(ROOT, "oracle", "fa_oracle.c"), str(tmp_path / "libfa_oracle_san.so"))
    gen = _build(tmp_path, os.path.join(ROOT, "synth", "gen.c"), str(tmp_path / "libsynth_san.so"))
    env = dict(os.environ)
    env["FA_ORACLE_LIB"] = orc
    env["FA_SYNTH_LIB"] = gen
    # the ASan runtime first, ahead of anything already preloaded
    env["LD_PRELOAD"] = ":".join(p for p in (asan, os.environ.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0:exitcode=97"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=98"
    env["OMP_NUM_THREADS"] = "4"
    script = tmp_path / "degenerate.py"
    script.write_text(f"ROOT = {ROOT!r}\n" + DEGENERATE)
    res = subprocess.run([sys.executable, str(script)], env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0 and "DEGENERATE_OK" in out, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    # the oracle's pins (worked example, closed forms, brute force, SDPA, streamed = materialised)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", "test_oracle_pin"],
                         env=env, capture_output=True, text=True, timeout=1200, cwd=ROOT)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
