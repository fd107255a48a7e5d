"""CPU checks of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments on the host before touching the GPU."""
import ctypes
import os
import re

import pytest

from block_drafting_verification_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsp.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsp_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("dsp_draft_markov_step", "dsp_tree_expand", "dsp_schedule_windows", "dsp_pack_ragged",
              "dsp_verify_rejection"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _abi.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _abi.SIGNATURES, f"binding lacks {name}"


def test_version_and_error_string():
    lib = _abi.load()
    assert lib.dsp_version() >> 16 >= 1
    assert isinstance(lib.dsp_last_error(), bytes)


def _err(rc):
    return rc, _abi.load().dsp_last_error().decode()


def test_host_validation_codes():
    lib = _abi.load()
    p = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation first
    # verify: K out of range, bad dtype, missing pointers, negative temperature, small workspace
    rc, msg = _err(lib.dsp_verify_rejection(p, 1, 100, p, p, 1, 700, 100, p, 7, None, 4, 65, 100, 0, 1.0, 0, 0,
                                            None, None, None, None, None, None, p, p, p, None, None, p, p, 1 << 30, None))
    assert rc == -2 and "K" in msg
    rc, _ = _err(lib.dsp_verify_rejection(p, 5, 100, p, p, 1, 700, 100, p, 7, None, 4, 7, 100, 0, 1.0, 0, 0,
                                          None, None, None, None, None, None, p, p, p, None, None, p, p, 1 << 30, None))
    assert rc == -3
    rc, _ = _err(lib.dsp_verify_rejection(p, 1, 100, None, p, 1, 700, 100, p, 7, None, 4, 7, 100, 0, 1.0, 0, 0,
                                          None, None, None, None, None, None, p, p, p, None, None, p, p, 1 << 30, None))
    assert rc == -1
    rc, _ = _err(lib.dsp_verify_rejection(p, 1, 100, p, p, 1, 700, 100, p, 7, None, 4, 7, 100, 0, -1.0, 0, 0,
                                          None, None, None, None, None, None, p, p, p, None, None, p, p, 1 << 30, None))
    assert rc == -2
    rc, _ = _err(lib.dsp_verify_rejection(p, 1, 100, p, p, 1, 700, 100, p, 7, p, 4, 7, 100, 0, 1.0, 0, 0,
                                          None, None, None, None, None, None, p, p, p, None, None, p, p, 1 << 30, None))
    assert rc == -6  # tree verify needs temperature 0
    rc, _ = _err(lib.dsp_verify_rejection(p, 1, 100, p, p, 1, 700, 100, p, 7, p, 4, 7, 100, 0, 0.0, 0, 0,
                                          None, None, None, None, p, None, p, p, p, None, None, p, p, 1 << 30, None))
    assert rc == -6  # cap-accept is chain-only
    rc, _ = _err(lib.dsp_verify_rejection(p, 1, 100, p, p, 1, 700, 100, p, 7, None, 4, 7, 100, 0, 1.0, 0, 0,
                                          None, None, None, None, None, None, p, p, p, None, None, p, p, 16, None))
    assert rc == -5
    big = 1 << 29  # a logit row of 2 GiB in fp32: past what the bounded row loads address
    rc, msg = _err(lib.dsp_verify_rejection(p, 1, big, p, p, 1, 7 * big, big, p, 7, None, 4, 7, big, 0, 1.0, 0, 0,
                                            None, None, None, None, None, None, p, p, p, None, None, p, p, 1 << 30,
                                            None))
    assert rc == -2 and "2 GiB" in msg
    # schedule + pack: the scheduler's limits, then the pack's pointers
    assert lib.dsp_schedule_pack(p, 9000, 1, p, 9001, 0, -1, 0.0, p, None, None, p, p, 1, None, 0, p, p, p, p, p,
                                 p, p, 1 << 20, None) == -2
    assert lib.dsp_schedule_pack(p, 4, 4, p, 17, 0, -1, 0.0, p, None, None, None, p, 4, None, 0, p, p, p, p, p,
                                 p, p, 1 << 20, None) == -1
    # schedule: too many candidates, short cost table, unknown mode
    assert lib.dsp_schedule_windows(p, 9000, 1, p, 9001, 0, -1, 0.0, p, None, None, None, 0, None) == -2
    assert lib.dsp_schedule_windows(p, 4, 4, p, 16, 0, -1, 0.0, p, None, None, None, 0, None) == -2
    assert lib.dsp_schedule_windows(p, 4, 4, p, 17, 4, -1, 0.0, p, None, None, None, 0, None) == -6
    assert lib.dsp_schedule_windows(p, 4, 4, p, 17, 3, -1, float('nan'), p, None, None, None, 0, None) == -2
    # schedule: the ranked keys need the queried workspace (in every mode)
    need = lib.dsp_schedule_windows_workspace_size(4, 4)
    assert need >= 4 * 4 * 8
    assert lib.dsp_schedule_windows(p, 4, 4, p, 17, 0, -1, 0.0, p, None, None, None, 0, None) == -5
    assert lib.dsp_schedule_windows(p, 4, 4, p, 17, 3, -1, 0.5, p, None, None, p, need - 1, None) == -5
    # pack: descending tiers, too many tiers
    tiers = (ctypes.c_int32 * 2)(8, 4)
    assert lib.dsp_pack_ragged(p, p, p, 4, 3, 4, ctypes.cast(tiers, ctypes.c_void_p), 2, p, p, p, p, p, p,
                               None) == -2
    assert lib.dsp_pack_ragged(p, p, p, 4, 3, 4, None, 65, p, p, p, p, p, p, None) == -2
    # markov: rank not a multiple of 32, misaligned factors
    assert lib.dsp_draft_markov_step(p, 1, 1000, 100, p, p, 100, 48, p, 2, 4, p, 4, None, p, p, 1 << 30,
                                     None) == -2
    assert lib.dsp_draft_markov_step(p, 1, 1000, 100, ctypes.c_void_p(18), p, 100, 64, p, 2, 4, p, 4, None,
                                     p, p, 1 << 30, None) == -4
    # markov, token-major base logits: rank 256 only, R a multiple of 8, strides and span
    TM = _abi.DSP_BF16_TOKEN_MAJOR
    assert lib.dsp_draft_markov_step(p, TM, 16, 16 * 100, p, p, 100, 64, p, 16, 4, p, 4, None, p, p, 1 << 30,
                                     None) == -6
    rc, msg = _err(lib.dsp_draft_markov_step(p, TM, 16, 16 * 100, p, p, 100, 256, p, 12, 4, p, 4, None, p, p,
                                             1 << 30, None))
    assert rc == -2 and "multiple of 8" in msg
    assert lib.dsp_draft_markov_step(p, TM, 8, 16 * 100, p, p, 100, 256, p, 16, 4, p, 4, None, p, p, 1 << 30,
                                     None) == -2  # token stride below R
    assert lib.dsp_draft_markov_step(p, TM, 16, 99 * 16, p, p, 100, 256, p, 16, 4, p, 4, None, p, p, 1 << 30,
                                     None) == -2  # depth stride below (V-1)*ldL_r + R
    assert lib.dsp_draft_markov_step(ctypes.c_void_p(24), TM, 16, 1600, p, p, 100, 256, p, 16, 4, p, 4, None, p,
                                     p, 1 << 30, None) == -4
    assert lib.dsp_draft_markov_step(p, TM, 20, 2000, p, p, 100, 256, p, 16, 4, p, 4, None, p, p, 1 << 30,
                                     None) == -4  # token stride not a multiple of 8
    rc, msg = _err(lib.dsp_draft_markov_step(p, TM, 1 << 14, 151936 << 14, p, p, 151936, 256, p, 16, 4, p, 4,
                                             None, p, p, 1 << 30, None))
    assert rc == -2 and "2 GiB" in msg
    assert lib.dsp_draft_markov_sample(p, TM, 12, 1200, p, p, 100, 256, p, 12, 4, 1.0, 0, 0, None, None, p, 4,
                                       None, p, 1000, 104, p, p, 1 << 30, None) == -2
    assert lib.dsp_tree_expand(p, TM, 16, 1600, p, p, 100, 256, p, 16, 4, 4, 4, 8, p, p, p, p, p, None, p, p,
                               1 << 30, None) == -6  # the tree takes row-major L
    # tree: top-k above 4
    assert lib.dsp_tree_expand(p, 1, 1000, 100, p, p, 100, 64, p, 2, 4, 5, 4, 8, p, p, p, p, p, None, p, p,
                               1 << 30, None) == -2
    # sampled chain: temperature 0 is the greedy entry point's; misaligned emitted rows
    assert lib.dsp_draft_markov_sample(p, 1, 1000, 100, p, p, 100, 64, p, 2, 4, 0.0, 0, 0, None, None, p, 4,
                                       None, p, 1000, 100, p, p, 1 << 30, None) == -2
    assert lib.dsp_draft_markov_sample(p, 1, 1000, 100, p, p, 100, 64, p, 2, 4, 1.0, 0, 0, None, None, p, 4,
                                       None, ctypes.c_void_p(24), 1000, 104, p, p, 1 << 30, None) == -4


def test_workspace_queries_are_pure_functions():
    lib = _abi.load()
    a = lib.dsp_verify_rejection_workspace_size(64, 7, 151936, 0, 1, 1)
    assert a == lib.dsp_verify_rejection_workspace_size(64, 7, 151936, 0, 1, 1) and a > 0
    assert lib.dsp_verify_rejection_workspace_size(0, 7, 10, 0, 1, 1) == 0
    assert lib.dsp_tree_expand_workspace_size(128, 16, 129280, 256, 4, 16, 64) > 0
    assert lib.dsp_draft_markov_step_workspace_size(256, 151936, 256, 16, 0) > 0


def test_options_match_the_header_and_are_checked():
    """The binding's option codes are the header's, every declared option is accepted and
    restored, and an undeclared code or a negative value is rejected (host only)."""
    src = open(HEADER).read()
    declared = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+(DSP_OPT_[A-Z_]+)\s+(\d+)", src)}
    assert declared
    for name, code in declared.items():
        assert getattr(_abi, name) == code, name
    err_shape = int(re.search(r"#define\s+DSP_ERR_SHAPE\s+(-?\d+)", src).group(1))
    lib = _abi.load()
    defaults = {"DSP_OPT_CHAIN_PERSISTENT": 0, "DSP_OPT_SPIN_LIMIT": 1 << 20, "DSP_OPT_TREE_SPLIT": 1,
                "DSP_OPT_CHAIN_SCHED": 0}
    assert set(defaults) == set(declared)
    for name, code in declared.items():
        assert lib.dsp_set_option(code, 0) == 0
        assert lib.dsp_set_option(code, -1) == err_shape
        assert lib.dsp_set_option(code, defaults[name]) == 0
    assert lib.dsp_set_option(max(declared.values()) + 1, 0) == err_shape
    assert lib.dsp_set_option(-1, 0) == err_shape
