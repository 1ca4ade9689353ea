"""The Python binding's argument marshalling (no library call, no device):
which gate-input forms it accepts, the shapes and dtypes it insists on, the
strides and pointers it writes into kda_decode_args, and that host tensors
are refused before any library call.

The marshalling checks run the binding's marshaller with the device every
tensor must be on set to the CPU (the library calls always pass torch's
current GPU), so that they need no GPU."""
import pytest
import torch

import linear_attention_recurrent_decode_amd as kda

CPU = torch.device("cpu")

T, H, HV, K, V, SLOTS = 3, 2, 4, 128, 128, 5


def _tensors():
    bf = torch.bfloat16
    return dict(
        q=torch.zeros((T, H, K), dtype=bf), k=torch.zeros((T, H, K), dtype=bf), v=torch.zeros((T, HV, V), dtype=bf),
        g=torch.zeros((T, HV, K)), beta=torch.zeros((T, HV)),
        state=torch.zeros((SLOTS, HV, K, V)), slot_idx=torch.zeros(T, dtype=torch.int32),
        out=torch.zeros((T, HV, V), dtype=bf),
        raw_gate=torch.zeros((T, HV, K), dtype=bf), raw_beta=torch.zeros((T, HV), dtype=bf),
        A_log=torch.zeros(HV), dt_bias=torch.zeros((HV, K)))


def _args(t, **kw):
    base = dict(q=t["q"], k=t["k"], v=t["v"], g=t["g"], beta=t["beta"], state=t["state"], slot_idx=t["slot_idx"],
                out=t["out"], scale=0.088, gate=None, norm_weight=None, eps=1e-6, device_status=None,
                inter_state=None, raw_gate=None, raw_beta=None, A_log=None, dt_bias=None)
    base.update(kw)
    return kda._marshal_args(**base, device=CPU)


@pytest.fixture
def no_library(monkeypatch):
    """Any attempt to load or call libkda.so fails the test."""
    def refuse():
        raise AssertionError("the library was reached")
    monkeypatch.setattr(kda, "library", refuse)


def test_host_tensors_are_refused_before_any_library_call(no_library):
    t = _tensors()
    with pytest.raises(ValueError, match="GPU tensor"):
        kda.kda_decode_step(t["q"], t["k"], t["v"], t["g"], t["beta"], t["state"], t["slot_idx"], t["out"],
                            T=1, scale=0.088)
    cu = torch.arange(T + 1, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        kda.kda_decode_packed(t["q"], t["k"], t["v"], t["g"], t["beta"], t["state"], t["slot_idx"], cu, t["out"],
                              scale=0.088)
    with pytest.raises(ValueError, match="GPU tensor"):
        kda.decode_args(t["q"], t["k"], t["v"], t["g"], t["beta"], t["state"], t["slot_idx"], t["out"], 0.088)
    x = torch.zeros((2, V), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        kda.kda_gated_rmsnorm(x, x.clone(), torch.ones(V, dtype=torch.bfloat16), x.clone())


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "state", "slot_idx", "out"])
def test_each_tensor_must_be_on_the_call_device(name):
    """One tensor on another device than the call's (here a meta tensor in a
    call whose device is the CPU) is refused, whichever it is."""
    t = _tensors()
    t[name] = t[name].to("meta")
    with pytest.raises(ValueError, match=f"{name} is on meta"):
        _args(t)


def test_activated_form():
    t = _tensors()
    a = _args(t)
    assert a.g == t["g"].data_ptr() and a.beta == t["beta"].data_ptr()
    assert not a.raw_gate and not a.raw_beta and not a.A_log and not a.dt_bias
    assert (a.g_stride, a.beta_stride, a.q_stride, a.slot_stride) == (HV * K, HV, H * K, HV * K * V)


def test_raw_form():
    t = _tensors()
    a = _args(t, g=None, beta=None, raw_gate=t["raw_gate"], raw_beta=t["raw_beta"], A_log=t["A_log"],
              dt_bias=t["dt_bias"])
    assert not a.g and not a.beta
    assert a.raw_gate == t["raw_gate"].data_ptr() and a.raw_beta == t["raw_beta"].data_ptr()
    assert a.A_log == t["A_log"].data_ptr() and a.dt_bias == t["dt_bias"].data_ptr()
    assert (a.raw_gate_stride, a.raw_beta_stride) == (HV * K, HV)


def test_raw_form_strided_rows():
    t = _tensors()
    wide = torch.zeros((T, HV * K + 64), dtype=torch.bfloat16)
    a = _args(t, g=None, beta=None, raw_gate=wide[:, :HV * K].view(T, HV, K), raw_beta=wide[:, -HV:],
              A_log=t["A_log"], dt_bias=t["dt_bias"])
    assert a.raw_gate_stride == HV * K + 64 and a.raw_beta_stride == HV * K + 64


@pytest.mark.parametrize("drop", ["raw_beta", "A_log", "dt_bias"])
def test_raw_form_is_all_or_nothing(drop):
    t = _tensors()
    kw = dict(g=None, beta=None, raw_gate=t["raw_gate"], raw_beta=t["raw_beta"], A_log=t["A_log"],
              dt_bias=t["dt_bias"])
    kw[drop] = None
    with pytest.raises(ValueError):
        _args(t, **kw)


def test_forms_do_not_mix():
    t = _tensors()
    with pytest.raises(ValueError):
        _args(t, raw_gate=t["raw_gate"], raw_beta=t["raw_beta"], A_log=t["A_log"], dt_bias=t["dt_bias"])
    with pytest.raises(ValueError):
        _args(t, A_log=t["A_log"])


@pytest.mark.parametrize("name,bad", [
    ("raw_gate", torch.zeros((T, HV, K))),                              # fp32, not bf16
    ("raw_beta", torch.zeros((T, HV))),
    ("A_log", torch.zeros(HV, dtype=torch.bfloat16)),
    ("dt_bias", torch.zeros((HV, K), dtype=torch.bfloat16)),
])
def test_raw_dtypes(name, bad):
    t = _tensors()
    kw = dict(g=None, beta=None, raw_gate=t["raw_gate"], raw_beta=t["raw_beta"], A_log=t["A_log"],
              dt_bias=t["dt_bias"])
    kw[name] = bad
    with pytest.raises(TypeError):
        _args(t, **kw)


@pytest.mark.parametrize("name,bad", [
    ("raw_gate", torch.zeros((T, HV, K // 2), dtype=torch.bfloat16)),
    ("raw_beta", torch.zeros((T, HV + 1), dtype=torch.bfloat16)),
    ("A_log", torch.zeros(HV + 1)),
    ("dt_bias", torch.zeros((HV, K + 1))),
])
def test_raw_shapes(name, bad):
    t = _tensors()
    kw = dict(g=None, beta=None, raw_gate=t["raw_gate"], raw_beta=t["raw_beta"], A_log=t["A_log"],
              dt_bias=t["dt_bias"])
    kw[name] = bad
    with pytest.raises(ValueError):
        _args(t, **kw)


def test_intermediate_state_shape_and_dtype():
    t = _tensors()
    a = _args(t, inter_state=torch.zeros((T, HV, K, V)))
    assert a.inter_stride == HV * K * V
    with pytest.raises(ValueError):
        _args(t, inter_state=torch.zeros((T + 1, HV, K, V)))
    with pytest.raises(TypeError):
        _args(t, inter_state=torch.zeros((T, HV, K, V), dtype=torch.bfloat16))   # must match the pool
