"""The C-ABI library loads, exports every function include/specdec.h declares, and rejects bad
host-side arguments before touching the GPU (these calls return before any HIP call, so they
run without a GPU)."""
import ctypes
import os
import pathlib
import re

import pytest

from speculative_decoding_verification_specdec_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "specdec.h")


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(specdec_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("specdec_verify", "specdec_verify_greedy", "specdec_verify_ex",
              "specdec_workspace_size", "specdec_status_string", "specdec_version",
              "specdec_ngram_propose", "specdec_ngram_workspace_size", "specdec_commit",
              "specdec_verify_match", "specdec_telemetry_update", "specdec_apply_k",
              "specdec_plan_k", "specdec_choose_k"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert lib.specdec_version() >= 100
    for s in range(-7, 1):
        assert lib.specdec_status_string(s)
    assert lib.specdec_status_string(-99) == b"unknown status"


def test_workspace_size(lib):
    assert lib.specdec_workspace_size(0, 5, 128256) == 0
    assert lib.specdec_workspace_size(-1, 5, 10) == 0
    assert lib.specdec_workspace_size(4, 64, 10) == 0          # K beyond the maximum
    a = lib.specdec_workspace_size(64, 5, 128256)
    b = lib.specdec_workspace_size(64, 5, 128256 * 2)
    assert 0 < a < b and a % 16 == 0


FAKE = 0x1000          # aligned, never dereferenced: every call below fails host-side checks


def _verify(lib, **kw):
    a = dict(logits=FAKE, dtype=1, q=FAKE, onehot=None, prop=FAKE, nd=None, T=FAKE, U=FAKE,
             B=4, K=3, V=64, acc=FAKE, tok=FAKE, prb=FAKE, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.specdec_verify(a["logits"], a["dtype"], a["q"], a["onehot"], a["prop"], a["nd"],
                              a["T"], a["U"], a["B"], a["K"], a["V"], a["acc"], a["tok"],
                              a["prb"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), -2), (dict(K=-1), -2), (dict(K=64), -2), (dict(V=0), -2),
    (dict(dtype=7), -3),
    (dict(logits=None), -1), (dict(acc=None), -1), (dict(tok=None), -1), (dict(ws=None), -1),
    (dict(prop=None), -1), (dict(T=None), -1), (dict(U=None), -1),
    (dict(logits=FAKE + 1), -4), (dict(q=FAKE + 2), -4), (dict(ws=FAKE + 8), -4),
    (dict(acc=FAKE + 2), -4),
    (dict(wsb=16), -5),
])
def test_host_side_errors(lib, kw, status):
    assert _verify(lib, **kw) == status


def _noalloc(lib, **kw):
    a = dict(logits=FAKE, dtype=1, q=FAKE, onehot=None, prop=FAKE, nd=None, T=FAKE, U=FAKE,
             B=4, K=3, V=64, acc=FAKE, tok=FAKE, prb=FAKE, stream=None)
    a.update(kw)
    return lib.specdec_verify_noalloc(a["logits"], a["dtype"], a["q"], a["onehot"], a["prop"],
                                      a["nd"], a["T"], a["U"], a["B"], a["K"], a["V"], a["acc"],
                                      a["tok"], a["prb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), -2), (dict(K=64), -2), (dict(V=0), -2), (dict(dtype=7), -3),
    (dict(logits=None), -1), (dict(acc=None), -1), (dict(tok=None), -1), (dict(prop=None), -1),
    (dict(T=None), -1), (dict(U=None), -1),
    (dict(logits=FAKE + 1), -4), (dict(q=FAKE + 2), -4), (dict(tok=FAKE + 2), -4),
    (dict(B=1 << 20, K=5, V=128256), -7),
])
def test_noalloc_host_side_errors(lib, kw, status):
    # The entry point without a workspace checks its arguments as specdec_verify does, and then
    # whether the workspace fits its built-in scratch, all before any HIP call.
    assert _noalloc(lib, **kw) == status


def test_noalloc_empty_batch_is_a_no_op(lib):
    assert _noalloc(lib, B=0, logits=None, acc=None, tok=None) == 0
    assert lib.specdec_noalloc_scratch_bytes() == 32 << 20


def test_path_option_errors(lib):
    # An unknown path, and the small-vocabulary path asked for a vocabulary above its limit, are shape
    # errors found before any launch.
    import ctypes
    from speculative_decoding_verification_specdec_amd.binding import (SPECDEC_PATH_QUAD,
                                                                       SPECDEC_PATH_SMALL_VOCAB,
                                                                       SPECDEC_SMALL_V_MAX,
                                                                       _Options)
    # Layout of specdec_options: two pointers, two int32, two pointers.
    assert ctypes.sizeof(_Options) == 40
    assert [(_Options.__dict__[f].offset) for f in ("hot_event_begin", "hot_event_end", "path",
                                                   "spin_limit", "draw_event_begin",
                                                   "draw_event_end")] == [0, 8, 16, 20, 24, 32]
    header = open(HEADER).read()
    assert f"#define SPECDEC_SMALL_V_MAX {SPECDEC_SMALL_V_MAX}" in header

    def ex(path, V):
        a = [FAKE, 1, FAKE, None, FAKE, None, FAKE, FAKE, 4, 3, V, FAKE, FAKE, FAKE, FAKE, 1 << 30,
             None]
        return lib.specdec_verify_ex(*a, ctypes.byref(_Options(None, None, path)))
    assert ex(5, 64) == -2 and ex(-1, 64) == -2
    assert ex(SPECDEC_PATH_SMALL_VOCAB, SPECDEC_SMALL_V_MAX + 1) == -2
    # The four-workgroups-per-sequence path takes rows of whole 16-byte vectors only (checked
    # before anything touches the device).
    assert ex(SPECDEC_PATH_QUAD, 20003) == -2


def test_empty_batch_is_a_no_op(lib):
    assert _verify(lib, B=0, logits=None, acc=None, tok=None, ws=None) == 0


def test_greedy_entry_point_errors(lib):
    g = lib.specdec_verify_greedy
    assert g(FAKE, 1, FAKE, None, 4, 3, 64, FAKE, FAKE, None, FAKE, 16, None) == -5
    assert g(FAKE, 1, None, None, 4, 3, 64, FAKE, FAKE, None, FAKE, 1 << 20, None) == -1
    assert g(FAKE + 1, 1, FAKE, None, 4, 3, 64, FAKE, FAKE, None, FAKE, 1 << 20, None) == -4


def _ngram(lib, **kw):
    a = dict(tok=FAKE, lens=FAKE, B=4, cap=100, n_min=1, n_max=4, K=5, prop=FAKE, nd=FAKE,
             ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.specdec_ngram_propose(a["tok"], a["lens"], a["B"], a["cap"], a["n_min"],
                                     a["n_max"], a["K"], a["prop"], a["nd"], a["ws"], a["wsb"],
                                     a["stream"])


def test_ngram_workspace_size(lib):
    assert lib.specdec_ngram_workspace_size(0, 100) == 0
    assert lib.specdec_ngram_workspace_size(3, 0) == 0
    assert lib.specdec_ngram_workspace_size(3, 8192) == 3 * 8
    assert lib.specdec_ngram_workspace_size(3, 8193) == 3 * 2 * 8


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), -2), (dict(cap=0), -2), (dict(K=-1), -2), (dict(K=64), -2),
    (dict(n_min=0), -2), (dict(n_min=3, n_max=2), -2), (dict(n_max=33), -2),
    (dict(tok=None), -1), (dict(lens=None), -1), (dict(nd=None), -1), (dict(ws=None), -1),
    (dict(prop=None), -1),
    (dict(tok=FAKE + 2), -4), (dict(prop=FAKE + 1), -4), (dict(ws=FAKE + 4), -4),
    (dict(wsb=4), -5),
])
def test_ngram_host_side_errors(lib, kw, status):
    assert _ngram(lib, **kw) == status


def test_ngram_empty_batch_and_k0(lib):
    assert _ngram(lib, B=0, tok=None, lens=None, nd=None, ws=None, prop=None) == 0


def _commit(lib, **kw):
    a = dict(acc=FAKE, out=FAKE, B=4, K=3, tok=FAKE, cap=100, sl=FAKE, tkv=None, dkv=None,
             pk=FAKE, off=FAKE, stream=None)
    a.update(kw)
    return lib.specdec_commit(a["acc"], a["out"], a["B"], a["K"], a["tok"], a["cap"], a["sl"],
                              a["tkv"], a["dkv"], a["pk"], a["off"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), -2), (dict(K=-1), -2), (dict(K=64), -2), (dict(cap=0), -2),
    (dict(acc=None), -1), (dict(out=None), -1), (dict(sl=None), -1),
    (dict(acc=FAKE + 1), -4), (dict(tok=FAKE + 2), -4), (dict(tkv=FAKE + 3), -4),
    (dict(off=FAKE + 2), -4),
])
def test_commit_host_side_errors(lib, kw, status):
    assert _commit(lib, **kw) == status


def test_commit_empty_batch_without_offsets(lib):
    assert _commit(lib, B=0, acc=None, out=None, sl=None, tok=None, pk=None, off=None) == 0


# ---- host arithmetic of the telemetry plan (no GPU needed): against the oracle ----

def test_host_plan_functions_match_the_oracle(lib):
    import json
    import numpy as np
    from oracle import closed_forms
    from oracle.telemetry_oracle import ROW, choose_k, plan_k
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "page1_speedup_tables.json")))
    lo, hi = g["best_k_search_range"]
    for c_str, tab in g["tables"].items():
        for alpha, (k_best, _) in zip(g["alphas"], tab["best"]):
            assert lib.specdec_choose_k(alpha, float(c_str), lo, hi) == k_best
    for alpha in np.linspace(0.0, 1.0, 21):
        for k in (0, 1, 5, 8, 63):
            assert lib.specdec_expected_tokens(alpha, k) == pytest.approx(
                closed_forms.expected_tokens(alpha, k), rel=1e-12)
            assert lib.specdec_speedup(alpha, k, 0.07) == pytest.approx(
                closed_forms.speedup(alpha, k, 0.07), rel=1e-12)
            assert lib.specdec_choose_k(alpha, 0.07, 0, k) == choose_k(alpha, 0.07, 0, k)
    rng = np.random.default_rng(4)
    cnt = np.zeros((9, ROW), dtype=np.int64)
    cnt[:, 2] = rng.integers(0, 5000, size=9)
    cnt[:, 5] = rng.integers(0, 5000, size=9)
    cnt[3, [2, 5]] = 0                                    # a route with no observations
    out = np.empty(9, dtype=np.int32)
    assert lib.specdec_plan_k(cnt.ctypes.data, 9, 0.1, 1, 12, 4, out.ctypes.data) == 0
    assert out.tolist() == plan_k(cnt, 0.1, 1, 12, 4).tolist()
    assert np.isnan(lib.specdec_alpha_estimate(cnt[3].ctypes.data))
    assert lib.specdec_alpha_estimate(cnt[0].ctypes.data) == cnt[0, 2] / (cnt[0, 2] + cnt[0, 5])


def test_host_plan_argument_errors(lib):
    import numpy as np
    assert lib.specdec_choose_k(1.5, 0.1, 1, 5) == -1
    assert lib.specdec_choose_k(0.5, -0.1, 1, 5) == -1
    assert lib.specdec_choose_k(0.5, 0.1, 5, 4) == -1
    assert lib.specdec_choose_k(0.5, 0.1, 1, 64) == -1
    cnt = np.zeros((2, 72), dtype=np.int64)
    out = np.empty(2, dtype=np.int32)
    assert lib.specdec_plan_k(cnt.ctypes.data, 0, 0.1, 1, 5, 3, out.ctypes.data) == -2
    assert lib.specdec_plan_k(None, 2, 0.1, 1, 5, 3, out.ctypes.data) == -1
    assert lib.specdec_plan_k(cnt.ctypes.data, 2, 0.1, 1, 5, 64, out.ctypes.data) == -2


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), -2), (dict(K=64), -2), (dict(n=0), -2), (dict(n=65), -2),
    (dict(acc=None), -1), (dict(cnt=None), -1),
    (dict(acc=FAKE + 1), -4), (dict(cnt=FAKE + 4), -4), (dict(route=FAKE + 2), -4),
])
def test_telemetry_host_side_errors(lib, kw, status):
    a = dict(acc=FAKE, nd=None, route=None, B=4, K=5, n=2, cnt=FAKE)
    a.update(kw)
    assert lib.specdec_telemetry_update(a["acc"], a["nd"], a["route"], a["B"], a["K"], a["n"],
                                        a["cnt"], None) == status


def test_apply_k_host_side_errors(lib):
    assert lib.specdec_apply_k(FAKE, None, FAKE, -1, 2, None) == -2
    assert lib.specdec_apply_k(FAKE, None, FAKE, 4, 0, None) == -2
    assert lib.specdec_apply_k(None, None, FAKE, 4, 2, None) == -1
    assert lib.specdec_apply_k(FAKE + 1, None, FAKE, 4, 2, None) == -4
    assert lib.specdec_apply_k(None, None, None, 0, 2, None) == 0


def test_missing_library_fails_loudly(tmp_path):
    # No CPU or PyTorch fallback: with the library absent the first call raises SpecdecError.
    # A fresh interpreter, since this process has the library loaded already.
    import subprocess
    import sys
    code = ("from speculative_decoding_verification_specdec_amd import SpecdecError, "
            "specdec_workspace_size\n"
            "try:\n"
            "    specdec_workspace_size(4, 2, 100)\n"
            "except SpecdecError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    raise SystemExit('no error')\n")
    env = dict(os.environ, SPECDEC_LIBRARY=str(tmp_path / "libspecdec_absent.so"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       cwd=str(pathlib.Path(__file__).resolve().parents[1]), timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "raised:" in r.stdout and "missing" in r.stdout
