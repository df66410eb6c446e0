"""Host logic of bench.py (no GPU): the method's byte and flop model, the
one-GPU guard, and the tie between recorded counters and the kernel sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_step_bytes_are_the_methods_own():
    """The 2 x 8192-token step with 16 key / 32 value heads, counted by hand:
    the forward reads q, k, v, g, beta and h0 and writes o, hT and the bf16
    per-chunk states; the backward reads q, k, v, g, beta, dO and those states
    and writes dq, dk, dv, dg, dbeta and dh0. Nothing else."""
    T, N, H, HV, NC = 16384, 2, 16, 32, 256
    bf, f32 = 2, 4
    q = k = T * H * 128 * bf
    v = o = dO = T * HV * 128 * bf
    g = beta = T * HV * f32
    state = N * HV * 128 * 128 * f32
    h_c = NC * HV * 128 * 128 * bf
    fwd = q + k + v + g + beta + state + o + state + h_c
    bwd = q + k + v + g + beta + dO + h_c + q + k + v + g + beta + state
    per, tot = bench.method_bytes(T, N, H, HV, NC)
    assert tot == {"fwd": fwd, "bwd": bwd, "step": fwd + bwd}
    assert tot["step"] == 1635778560
    # every kernel's share is part of its pass's bytes; the gradient pass
    # needs the whole backward except the dh scan's dh0
    assert per["chunk_prep"] + per["fwd_scan"] == fwd
    assert per["bwd_chunk"] == bwd - state
    assert per["bwd_dh_scan"] <= bwd


def test_flop_model():
    """Per chunk and value head: the strictly lower K K^T, the triangular
    solve, four lower-triangular 64 x 64 by 64 x 128 products and three state
    products (the chunk form's forward); forward + backward is three times it,
    and the per-kernel shares add up to it."""
    C, D = 64, 128
    f = C * (C - 1) * D + C ** 3 // 3 + 4 * C * (C + 1) * D + 3 * 2 * C * D * D
    assert bench.F_FWD == f == 9024853
    assert sum(bench.KERNEL_FLOPS.values()) == 3 * bench.F_FWD


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_recorded_counters_follow_the_kernel_sources(tmp_path, monkeypatch):
    """Counters recorded for other kernel sources are not reported."""
    text = open(os.path.join(ROOT, "profiles", bench.WORKLOAD + ".md")).read()
    blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    assert set(bench.STAGE_KERNELS.values()) <= set(blob["kernels"])
    prof = tmp_path / "profiles"
    prof.mkdir()
    stale = dict(blob, source="0" * 16)
    (prof / (bench.WORKLOAD + ".md")).write_text("```json\n" + json.dumps(stale) + "\n```\n")
    real_root = bench.ROOT
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_counters() == {}
    fresh = dict(blob)
    monkeypatch.setattr(bench, "ROOT", real_root)
    fresh["source"] = bench.kernel_source_hash()
    (prof / (bench.WORKLOAD + ".md")).write_text("```json\n" + json.dumps(fresh) + "\n```\n")
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: fresh["source"])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_counters() == blob["kernels"]


@pytest.mark.parametrize("section", ["step", "fwd", "decode", "paged", "recompute", "conv"])
def test_profile_sections_are_offered(section):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and section in r.stdout


def test_source_hash_ignores_comments_but_not_code():
    """A comment edit keeps recorded counters valid; a code edit voids them."""
    base = "int f(int a) { return a + 1; } // one\n/* two */ const char* s = \"// x\";\n"
    same = "int f(int a)   {\n  return a + 1;   }  // edited\nconst char* s = \"// x\"; /* new */\n"
    code = base.replace("a + 1", "a + 2")
    lit = base.replace("\"// x\"", "\"// y\"")
    assert bench._code_tokens(base) == bench._code_tokens(same)
    assert bench._code_tokens(base) != bench._code_tokens(code)
    assert bench._code_tokens(base) != bench._code_tokens(lit)
