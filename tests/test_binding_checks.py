"""The Python binding refuses, before any library call, tensors the kernels
would read or write out of bounds: host tensors passed as device arguments,
wrong element types, and sizes or counts beyond the tensors (no GPU needed)."""
import pytest
import torch

HP = dict(lr=3e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=1.0)


@pytest.fixture(scope="module")
def zf():
    import fsdp_sharded_mixed_flatparameter_amd as m
    return m


def test_host_tensors_are_not_device_arguments(zf):
    t16 = torch.zeros(64, dtype=torch.float16)
    t32 = torch.zeros(64)
    with pytest.raises(ValueError, match="device"):
        zf.zero_grad_reduce_shard([t16, t16], 0, 64, zf.ZERO_AVG, t32)
    with pytest.raises(ValueError, match="device"):
        zf.zero_unscale_norm(t16, None)
    with pytest.raises(ValueError, match="device"):
        zf.zero_adamw_shard_step(t16, t32, t32, t32, t16, 0, HP, None)
    with pytest.raises(ValueError, match="device"):
        zf.zero_quant_allgather_slot(t16, torch.zeros(64, dtype=torch.int8), torch.zeros(1))
    with pytest.raises(ValueError, match="device"):
        zf.zero_dequant_allgather(torch.zeros(64, dtype=torch.int8), torch.zeros(1), 1, 64, t16)
    with pytest.raises(ValueError, match="device"):
        zf.zero_grad_reduce_shard_int8([torch.zeros(64, dtype=torch.int8)], [torch.zeros(1)], 64,
                                       zf.ZERO_AVG, t32)


def test_wrong_element_types_are_refused(zf):
    t = torch.zeros(16)
    lp = torch.zeros(16, dtype=torch.float16)
    st = zf.zero_step_state_init(1.0, False)
    with pytest.raises(ValueError, match="float32"):
        zf.zero_offload_adamw_host(t, lp, t, t, lp, HP, st)         # fp16 master


def test_sizes_beyond_tensors_are_refused(zf):
    t = torch.zeros(16)
    lp = torch.zeros(16, dtype=torch.float16)
    st = zf.zero_step_state_init(1.0, False)
    with pytest.raises(ValueError):
        zf.zero_offload_adamw_host(t[:8], t, t, t, lp, HP, st)      # gradient too short
    with pytest.raises(ValueError):
        zf.unflatten(torch.zeros(10), [(4, 4)])
