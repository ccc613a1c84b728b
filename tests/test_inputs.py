"""The seeded input generators: deterministic, right shapes, P and P_cols agree."""

import torch

from transformer_attention_query_amd import inputs as tinputs


def test_same_seed_same_bytes():
    a = tinputs.make_prefill_inputs(1, 33, 4, 2, 128, 32, 16, "bf16", seed=7)
    b = tinputs.make_prefill_inputs(1, 33, 4, 2, 128, 32, 16, "bf16", seed=7)
    for n in a:
        assert torch.equal(a[n].view(torch.int16) if a[n].dtype == torch.bfloat16 else a[n],
                           b[n].view(torch.int16) if b[n].dtype == torch.bfloat16 else b[n])
    c = tinputs.make_prefill_inputs(1, 33, 4, 2, 128, 32, 16, "bf16", seed=8)
    assert not torch.equal(a["q"].float(), c["q"].float())


def test_shapes_and_P_layout():
    w = tinputs.WORKLOADS["tiny_fp32"]
    x = tinputs.make_inputs(w)
    assert x["q"].shape == (1, 256, 4, 128) and x["q"].dtype == torch.float32
    assert x["k"].shape == (1, 256, 1, 128) and x["r"].shape == (1, 256, 4, 32)
    assert x["P"].shape == (32, 64) and x["P_cols"].shape == (64, 32)
    assert x["P_cols"].is_contiguous()
    assert torch.equal(x["P_cols"], x["P"].t())
    # P ~ N(0, 0.02^2): sample std close to 0.02
    assert abs(x["P"].std().item() - 0.02) < 0.003
    d = tinputs.make_decode_inputs(3, 50, 16, 2, 128, 128, 64, "bf16")
    assert d["q"].shape == (3, 16, 128) and d["k"].shape == (3, 50, 2, 128) and d["r"].shape == (3, 16, 128)


def test_workload_table_matches_spec():
    W = tinputs.WORKLOADS
    assert (W["swa_prefill_8k"].T, W["swa_prefill_8k"].W, W["swa_prefill_8k"].E) == (8192, 1024, 1024)
    assert W["full_prefill_32k_log"].B == 2 and W["full_prefill_32k_log"].log_scale
    assert W["decode_1x1m_log"].T == 1048576 and W["decode_64x8k"].B == 64
    for w in W.values():
        assert w.D == 128 and w.Hq % w.Hkv == 0


def test_backward_inputs_extend_the_prefill_draws():
    """The backward recipe draws the prefill tensors first, so they equal the
    prefill inputs of the same seed; dout comes last."""
    a = tinputs.make_prefill_inputs(1, 40, 4, 2, 128, 32, 16, "bf16", seed=3)
    b = tinputs.make_backward_inputs(1, 40, 4, 2, 128, 32, 16, "bf16", seed=3)
    for n in a:
        assert torch.equal(a[n].float(), b[n].float())
    assert b["dout"].shape == (1, 40, 4, 128) and b["dout"].dtype == torch.bfloat16
    w = tinputs.WORKLOADS["swa_backward_8k"]
    assert (w.kind, w.T, w.W, w.E, w.d_r) == ("backward", 8192, 1024, 1024, 128)
