"""CPU checks of the autograd wrappers' argument rules (raised before any device call)."""
import pytest
import torch

from linear_cross_entropy_masked_amd import autograd as ag


def test_reduction_rules():
    z = torch.zeros(4, 8, dtype=torch.bfloat16)
    y = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError, match="reduction"):
        ag.masked_cross_entropy(z, y, reduction="avg")
    with pytest.raises(ValueError, match="num_label_tokens"):
        ag.masked_cross_entropy(z, y, reduction="mean", num_label_tokens=3)
    with pytest.raises(ValueError, match="num_label_tokens"):
        ag.masked_cross_entropy(z, y, reduction="none", num_label_tokens=3)
    with pytest.raises(ValueError, match="reduction"):
        ag.MaskedCrossEntropy(reduction="max")
    with pytest.raises(ValueError, match="reduction"):
        ag.linear_cross_entropy(torch.zeros(4, 8, dtype=torch.bfloat16),
                                torch.zeros(5, 8, dtype=torch.bfloat16), y, reduction="none")
    with pytest.raises(ValueError, match="reduction"):
        ag.LinearCrossEntropy(reduction="none")


def test_shape_rules():
    z = torch.zeros(2, 3, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="labels has"):
        ag.masked_cross_entropy(z, torch.zeros(5, dtype=torch.int64))
    with pytest.raises(ValueError, match="mask has"):
        ag.masked_cross_entropy(z, torch.zeros(2, 3, dtype=torch.int64),
                                mask=torch.ones(7, dtype=torch.bool))
    with pytest.raises(ValueError, match="weight_grad_buffer"):
        ag.linear_cross_entropy(torch.zeros(4, 8, dtype=torch.bfloat16),
                                torch.zeros(5, 8, dtype=torch.bfloat16),
                                torch.zeros(4, dtype=torch.int64),
                                weight_grad_buffer=torch.zeros(5, 8, dtype=torch.bfloat16))


def test_host_tensors_are_refused_not_computed():
    """No CPU fallback: host tensors are rejected by the binding."""
    z = torch.zeros(4, 8, dtype=torch.bfloat16)
    y = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError, match="HIP device"):
        ag.masked_cross_entropy(z, y)


def test_normaliser_mapping():
    assert ag._normaliser("sum", None) == 1
    assert ag._normaliser("sum", 37) == 37
    assert ag._normaliser("mean", None) == -1


def test_interface_aliases():
    with pytest.raises(ValueError, match="recomputes"):
        ag.flce(torch.zeros(4, 8, dtype=torch.bfloat16), torch.zeros(5, 8, dtype=torch.bfloat16),
                torch.zeros(4, dtype=torch.int64), recompute=False)
    assert ag.ce_chunked.__name__ == "ce_chunked" and ag.flce.__name__ == "flce"
