"""ctypes declarations of libdsp's C ABI (the functions declared in include/dsp.h)."""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsp.so")

DSP_OK = 0
DSP_F32 = 0
DSP_BF16 = 1
DSP_BF16_TOKEN_MAJOR = 2
DSP_STATUS_TOKEN_RANGE = 1
DSP_STATUS_WINDOW_RANGE = 2
DSP_STATUS_NONFINITE = 4
DSP_STATUS_TIMEOUT = 8
DSP_OPT_CHAIN_PERSISTENT = 0
DSP_OPT_SPIN_LIMIT = 1
DSP_OPT_TREE_SPLIT = 2
DSP_OPT_CHAIN_SCHED = 3
DSP_SCHED_EARLY_STOP = 0
DSP_SCHED_ARGMAX = 1
DSP_SCHED_TOP_M = 2
DSP_SCHED_THRESHOLD = 3

KERNELS = ["VERIFY_STATS", "VERIFY_DECIDE", "VERIFY_RESIDUAL", "VERIFY_SAMPLE", "SCHEDULE", "PACK",
           "MARKOV_GEMM", "MARKOV_MERGE", "TREE_GEMM", "TREE_MERGE", "TREE_FINAL", "SCHEDULE_RANK", "CONFIDENCE",
           "TREE_PROBE", "CALIBRATION", "RNN_MEMO", "RNN_PROJ", "CHAIN_PERSIST"]

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64
_sz = ctypes.c_size_t
_f32 = ctypes.c_float

SIGNATURES = {
    "dsp_version": (_i32, []),
    "dsp_last_error": (ctypes.c_char_p, []),
    "dsp_philox_uniforms": (_i32, [_p, _i64, _u64, _p, _p]),
    "dsp_verify_calibration": (_i32, [_p, _i64, _p, _p, _i32, _i32, _i32, _p, _p, _p, _p]),
    "dsp_confidence_head": (_i32, [_p, _i32, _i64, _i64, _p, _i32, _f32, _p, _i32, _i32, _i32, _p, _p, _p]),
    "dsp_schedule_windows_workspace_size": (_sz, [_i32, _i32]),
    "dsp_schedule_windows": (_i32, [_p, _i32, _i32, _p, _i32, _i32, _i32, ctypes.c_double, _p, _p, _p, _p, _sz,
                                    _p]),
    "dsp_pack_ragged": (_i32, [_p, _p, _p, _i64, _i32, _i32, _p, _i32, _p, _p, _p, _p, _p, _p, _p]),
    "dsp_schedule_pack": (_i32, [_p, _i32, _i32, _p, _i32, _i32, _i32, ctypes.c_double, _p, _p, _p, _p, _p, _i64, _p,
                                 _i32, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "dsp_verify_rejection_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "dsp_verify_rejection": (_i32, [_p, _i32, _i64, _p, _p, _i32, _i64, _i64, _p, _i64, _p,
                                    _i32, _i32, _i32, _i32, _f32, _u64, _u64, _p, _p, _p, _p, _p, _p,
                                    _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "dsp_verify_rejection_noalloc": (_i32, [_p, _i32, _i64, _p, _p, _i32, _i64, _i64, _p, _i64, _p,
                                            _i32, _i32, _i32, _i32, _f32, _u64, _u64, _p, _p, _p, _p, _p, _p,
                                            _p, _p, _p, _p, _p, _p, _p]),
    "dsp_draft_rnn_step_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "dsp_draft_rnn_step": (_i32, [_p, _i32, _i64, _i64, _p, _i32, _i64, _i64, _i32, _p, _p, _p, _p, _p, _i32, _i32,
                                  _p, _i32, _i32, _p, _i64, _p, _p, _p, _sz, _p]),
    "dsp_draft_markov_step_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "dsp_draft_markov_step": (_i32, [_p, _i32, _i64, _i64, _p, _p, _i32, _i32, _p, _i32, _i32,
                                     _p, _i64, _p, _p, _p, _sz, _p]),
    "dsp_draft_markov_sample_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "dsp_draft_markov_sample": (_i32, [_p, _i32, _i64, _i64, _p, _p, _i32, _i32, _p, _i32, _i32, _f32, _u64, _u64,
                                       _p, _p, _p, _i64, _p, _p, _i64, _i64, _p, _p, _sz, _p]),
    "dsp_tree_expand_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "dsp_tree_expand": (_i32, [_p, _i32, _i64, _i64, _p, _p, _i32, _i32, _p, _i32, _i32, _i32,
                               _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "dsp_stream_read": (_i32, [_p, _sz, _p, _p]),
    "dsp_prof_enable": (_i32, [_i32]),
    "dsp_set_option": (_i32, [_i32, _i64]),
    "dsp_prof_reset": (_i32, []),
    "dsp_prof_query": (_i32, [_i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
}

_lib = None


class DspError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libdsp error {code}: {msg}")
        self.code = code


def load():
    """Load libdsp.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_drafting_verification_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(rc):
    if rc != DSP_OK:
        raise DspError(rc, load().dsp_last_error().decode())
    return rc
