"""The Python binding refuses, before any call into the library, tensors that
the C ABI would read or write out of bounds or misread: a wrong dtype or shape,
a non-contiguous view, tensors on different devices, or tensors off the GPU.
(CPU tensors; no GPU needed.)"""
import pytest
import torch

from mhc_hyper_connection_boundary_amd import api

T, D = 8, 256
f32, bf16 = torch.float32, torch.bfloat16


def valid():
    return dict(x=torch.zeros(T, D, dtype=bf16), residual=torch.zeros(T, 4, D, dtype=bf16),
                post_prev=torch.zeros(T, 4), comb_prev=torch.zeros(T, 4, 4),
                pre_lag=torch.zeros(T, 4), w_prepared=torch.zeros(384 * D, dtype=torch.uint8),
                scale=torch.zeros(3), base=torch.zeros(24), norm_w=torch.zeros(D, dtype=bf16))


def call_boundary(a, **kw):
    return api.boundary(a["x"], a["residual"], a["post_prev"], a["comb_prev"], a["pre_lag"],
                        a["w_prepared"], a["scale"], a["base"], a["norm_w"], **kw)


BAD = [
    ("x", torch.zeros(T, D, dtype=f32), "x must be torch.bfloat16"),
    ("x", torch.zeros(T, D + 8, dtype=bf16), "x must have shape"),
    ("x", torch.zeros(D, T, dtype=bf16).t(), "x must be contiguous"),
    ("residual", torch.zeros(T, 4, D, dtype=f32), "residual must be torch.bfloat16"),
    ("post_prev", torch.zeros(T + 1, 4), "post_prev must have shape"),
    ("post_prev", torch.zeros(T, 4, dtype=torch.float64), "post_prev must be torch.float32"),
    ("comb_prev", torch.zeros(T, 4, 4).transpose(1, 2), "comb_prev must be contiguous"),
    ("comb_prev", torch.zeros(T, 16), "comb_prev must have shape"),
    ("pre_lag", torch.zeros(T - 1, 4), "pre_lag must have shape"),
    ("w_prepared", torch.zeros(384 * D - 16, dtype=torch.uint8), "w_prepared must have shape"),
    ("scale", torch.zeros(4), "scale must have shape"),
    ("base", torch.zeros(24, dtype=bf16), "base must be torch.float32"),
    ("norm_w", torch.zeros(D // 2, dtype=bf16), "norm_w must have shape"),
    ("x", torch.zeros(T, D, dtype=bf16, device="meta"), "expected cpu"),
]


@pytest.mark.parametrize("name,tensor,msg", BAD)
def test_boundary_refuses(name, tensor, msg):
    a = valid()
    a[name] = tensor
    with pytest.raises(ValueError, match=msg):
        call_boundary(a)


def test_boundary_refuses_bad_out_and_workspace():
    a = valid()
    with pytest.raises(ValueError, match="out\\['layer_input'\\] must have shape"):
        call_boundary(a, out=dict(layer_input=torch.zeros(T, D + 1, dtype=bf16)))
    with pytest.raises(ValueError, match="out\\['pre'\\] must be torch.float32"):
        call_boundary(a, out=dict(pre=torch.zeros(T, 4, dtype=bf16)))


def test_valid_cpu_tensors_are_refused_as_off_gpu():
    with pytest.raises(ValueError, match="must be on a GPU"):
        call_boundary(valid())
    a = valid()
    with pytest.raises(ValueError, match="must be on a GPU"):
        api.pre(a["residual"], a["w_prepared"], a["scale"], a["base"], a["norm_w"])
    with pytest.raises(ValueError, match="must be on a GPU"):
        api.post(a["x"], a["residual"], a["post_prev"], a["comb_prev"])
    with pytest.raises(ValueError, match="must be on a GPU"):
        api.pre_mixes(a["residual"], torch.zeros(2, T, 24), torch.zeros(2, T), a["scale"],
                      a["base"], a["norm_w"])
    with pytest.raises(ValueError, match="must be on a GPU"):
        api.prepare_weight(torch.zeros(24, 4 * D))
    with pytest.raises(ValueError, match="must be on a GPU"):
        api.prefetch_weight(a["w_prepared"], D)


def test_other_entry_points_refuse():
    a = valid()
    with pytest.raises(ValueError, match="residual must be a \\[T, 4, hidden\\] tensor"):
        api.pre(torch.zeros(T, 3, D, dtype=bf16), a["w_prepared"], a["scale"], a["base"])
    with pytest.raises(ValueError, match="w_prepared must have shape"):
        api.pre(a["residual"], a["w_prepared"][:-16], a["scale"], a["base"])
    with pytest.raises(ValueError, match="sqrsum must have shape"):
        api.pre_mixes(a["residual"], torch.zeros(2, T, 24), torch.zeros(3, T), a["scale"], a["base"])
    with pytest.raises(ValueError, match="dot_mix must be"):
        api.pre_mixes(a["residual"], torch.zeros(2, T, 24, dtype=bf16), torch.zeros(2, T),
                      a["scale"], a["base"])
    with pytest.raises(ValueError, match="out must have shape"):
        api.post(a["x"], a["residual"], a["post_prev"], a["comb_prev"],
                 out=torch.zeros(T, 4, D - 8, dtype=bf16))
    with pytest.raises(ValueError, match="w must be a \\[24, 4\\*hidden\\] tensor"):
        api.prepare_weight(torch.zeros(23, 4 * D))
    with pytest.raises(ValueError, match="w must be torch.float32"):
        api.prepare_weight(torch.zeros(24, 4 * D, dtype=torch.float64))
    with pytest.raises(ValueError, match="w_prepared must have shape"):
        api.prefetch_weight(a["w_prepared"], 2 * D)
