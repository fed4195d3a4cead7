"""The binding's argument checks that need no GPU: weight parts that disagree, activations and
weights of different dtypes, and host tensors where the library needs device memory are refused
before any pointer reaches the C entry points."""
import pytest

torch = pytest.importorskip("torch")
b = pytest.importorskip("post_quantization_mean_amd.binding")


def test_parts_must_agree():
    w = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="no weight parts"):
        b._parts([])
    with pytest.raises(ValueError, match="d_in"):
        b._parts([w, torch.zeros((4, 384), dtype=torch.bfloat16)])
    with pytest.raises(ValueError, match="dtype"):
        b._parts([w, torch.zeros((4, 256), dtype=torch.float32)])
    with pytest.raises(ValueError, match="contiguous"):
        b._parts([torch.zeros((256, 4), dtype=torch.bfloat16).t()])
    with pytest.raises(TypeError, match="must agree"):
        b._parts([w], torch.float32)


def test_host_tensors_are_refused():
    with pytest.raises(ValueError, match="device tensor"):
        b._parts([torch.zeros((4, 256), dtype=torch.bfloat16)])  # dtype and d_in agree: the device check fires
    with pytest.raises(ValueError, match="device tensor"):
        b._buf(torch.zeros(8, dtype=torch.float64), "act_mean", torch.float64, 8)
    with pytest.raises(ValueError, match="device tensor"):
        b._x_args(torch.zeros((8, 256), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="matrix"):
        b._x_args(torch.zeros(8, dtype=torch.bfloat16))


def test_block_level_calls_take_bfloat16_activations():
    with pytest.raises(TypeError, match="bfloat16"):
        b._x_bf16(torch.zeros((8, 256), dtype=torch.float32))
