"""Host-side checks of the step driver (CPU only): every workload and mode
builds its buffers and plans on the host, and its first call is refused by the
binding's operand checks (CPU tensors), so nothing reaches a kernel."""
import dataclasses

import pytest

from tp_inputs import get_config, make_inputs


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}), ("gpt2s", {}), ("gpt2s", {"recompute": True}), ("gpt2s", {"fused_bwd": False}),
    ("gpt2s", {"fp8": True}), ("attn", {}), ("attn", {"attn_core": True}),
    ("gpt350m", {"attn_core": True}), ("gpt175b", {}),
])
def test_step_builds_on_the_host_and_the_binding_refuses_cpu_tensors(name, kw):
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = get_config(name)
    if name == "gpt175b":
        cfg = dataclasses.replace(cfg, h=512, seq=256)
    elif cfg.T > 1024:
        cfg = dataclasses.replace(cfg, micro_batch=1, seq=256)
    step = ShardStep(cfg, make_inputs(cfg), "cpu", **kw)
    assert step.out and step.workspace.numel() >= 16
    with pytest.raises(ValueError, match="GPU tensor"):
        step.run_eager()
