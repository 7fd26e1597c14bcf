"""Host-side argument checks of the Python binding and the C validator of sequence offsets.

The kernels trust every size they are given, so a wrongly shaped tensor must be rejected before
any launch: these tests pass CPU tensors and expect ValueError / AttnSinkError from the checks
alone (no GPU is needed, and nothing reaches a kernel)."""
import ctypes
import os

import pytest
import torch

import attention_learnable_sinks_attn_amd as asa

needs_lib = pytest.mark.skipif(not os.path.exists(asa.library_path()),
                               reason="libattn_sink.so not built (python -m attention_learnable_sinks_attn_amd.build)")

T, HQ, HKV, D = 40, 8, 2, 64


def tensors(**over):
    t = dict(q=torch.zeros(T, HQ, D, dtype=torch.bfloat16), k=torch.zeros(T, HKV, D, dtype=torch.bfloat16),
             v=torch.zeros(T, HKV, D, dtype=torch.bfloat16), sinks=torch.zeros(HQ),
             cu=torch.tensor([0, 10, T], dtype=torch.int32), out=torch.zeros(T, HQ, D), lse=torch.zeros(HQ, T),
             dout=torch.zeros(T, HQ, D, dtype=torch.bfloat16), dq=torch.zeros(T, HQ, D),
             dk=torch.zeros(T, HKV, D), dv=torch.zeros(T, HKV, D), dsinks=torch.zeros(HQ))
    t.update(over)
    return t


def call_fwd(**over):
    t = tensors(**over)
    return asa.fwd(t["q"], t["k"], t["v"], t["sinks"], t["cu"], 30, out=t["out"], lse=t["lse"])


def call_bwd(**over):
    t = tensors(**over)
    return asa.bwd(t["q"], t["k"], t["v"], t["sinks"], t["out"], t["lse"], t["dout"], t["cu"], 30, dq=t["dq"],
                   dk=t["dk"], dv=t["dv"], dsinks=t["dsinks"])


BAD_FWD = {
    "k_head_dim": dict(k=torch.zeros(T, HKV, 32, dtype=torch.bfloat16)),
    "k_tokens": dict(k=torch.zeros(T + 1, HKV, D, dtype=torch.bfloat16)),
    "v_heads": dict(v=torch.zeros(T, HKV + 1, D, dtype=torch.bfloat16)),
    "gqa_ratio": dict(k=torch.zeros(T, 3, D, dtype=torch.bfloat16), v=torch.zeros(T, 3, D, dtype=torch.bfloat16)),
    "sinks_len": dict(sinks=torch.zeros(HQ - 1)),
    "q_2d": dict(q=torch.zeros(T, HQ * D, dtype=torch.bfloat16)),
    "cu_2d": dict(cu=torch.zeros(1, 3, dtype=torch.int32)),
    "cu_short": dict(cu=torch.zeros(1, dtype=torch.int32)),
    "out_shape": dict(out=torch.zeros(T, HQ, D + 1)),
    "lse_transposed": dict(lse=torch.zeros(T, HQ)),
}


@needs_lib
@pytest.mark.parametrize("case", list(BAD_FWD))
def test_forward_rejects_bad_shapes(case):
    with pytest.raises(ValueError):
        call_fwd(**BAD_FWD[case])


BAD_BWD = dict(BAD_FWD)
BAD_BWD.update({
    "dout_shape": dict(dout=torch.zeros(T, HQ, D - 1, dtype=torch.bfloat16)),
    "dq_shape": dict(dq=torch.zeros(T, HKV, D)),
    "dk_shape": dict(dk=torch.zeros(T, HQ, D)),
    "dv_tokens": dict(dv=torch.zeros(T - 1, HKV, D)),
    "dsinks_len": dict(dsinks=torch.zeros(HQ + 1)),
})
del BAD_BWD["out_shape"]
BAD_BWD["out_shape"] = dict(out=torch.zeros(T, HQ - 1, D))


@needs_lib
@pytest.mark.parametrize("case", list(BAD_BWD))
def test_backward_rejects_bad_shapes(case):
    with pytest.raises(ValueError):
        call_bwd(**BAD_BWD[case])


@needs_lib
def test_decode_rejects_bad_shapes():
    q = torch.zeros(3, HQ, D, dtype=torch.bfloat16)
    k = torch.zeros(50, HKV, D, dtype=torch.bfloat16)
    cq = torch.tensor([0, 1, 3], dtype=torch.int32)
    ck = torch.tensor([0, 20, 50], dtype=torch.int32)
    with pytest.raises(ValueError):  # v does not match k
        asa.decode_fwd(q, k, torch.zeros(50, HKV, 32, dtype=torch.bfloat16), torch.zeros(HQ), cq, ck, 2, 30)
    with pytest.raises(ValueError):  # one offset array per sequence count
        asa.decode_fwd(q, k, k.clone(), torch.zeros(HQ), cq, torch.tensor([0, 50], dtype=torch.int32), 2, 50)
    with pytest.raises(ValueError):
        asa.decode_fwd(q, k, k.clone(), torch.zeros(HQ), cq, ck, 2, 30, lse=torch.zeros(3, HQ))


def check(cu, T_, maxlen):
    arr = (ctypes.c_int32 * len(cu))(*cu)
    return asa.load_library().attn_sink_check_cu_seqlens(ctypes.cast(arr, ctypes.c_void_p), len(cu) - 1, T_, maxlen)


@needs_lib
def test_c_validator_of_sequence_offsets():
    assert check([0, 10, 10, 40], 40, 30) == 0
    assert check([0, 40], 40, 40) == 0
    assert check([0, 0], 0, 0) == 0
    assert check([1, 10, 40], 40, 30) == -8     # does not start at 0
    assert check([0, 10, 39], 40, 30) == -8     # does not end at T
    assert check([0, 20, 10, 40], 40, 30) == -8  # decreasing
    assert check([0, 10, 40], 40, 29) == -8     # a sequence longer than max_seqlen (rows left unwritten)
    assert check([0, 10, 40], 40, -1) == -2
    assert asa.load_library().attn_sink_check_cu_seqlens(None, 1, 0, 0) == -1
    arr = (ctypes.c_int32 * 1)(0)
    assert asa.load_library().attn_sink_check_cu_seqlens(ctypes.cast(arr, ctypes.c_void_p), 0, 0, 0) == -2


@needs_lib
def test_binding_validator_raises_before_launch():
    cu = torch.tensor([0, 10, T], dtype=torch.int32)
    asa.check_cu_seqlens(cu, T, 30)
    with pytest.raises(asa.AttnSinkError) as e:
        asa.check_cu_seqlens(cu, T, 29)
    assert e.value.code == -8
    t = tensors()
    with pytest.raises(asa.AttnSinkError):
        asa.fwd(t["q"], t["k"], t["v"], t["sinks"], cu, 29, out=t["out"], lse=t["lse"], validate_seqlens=True)
    with pytest.raises(asa.AttnSinkError):
        asa.bwd(t["q"], t["k"], t["v"], t["sinks"], t["out"], t["lse"], t["dout"], torch.tensor([0, 5, T - 1],
                dtype=torch.int32), 30, dq=t["dq"], dk=t["dk"], dv=t["dv"], dsinks=t["dsinks"],
                validate_seqlens=True)
