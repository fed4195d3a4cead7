"""The Python binding refuses arguments the C entry points cannot check (they receive bare
pointers): a wrong dtype, a short or strided buffer, weight parts that disagree, activations and
weights of different dtypes. Every case raises before any kernel is launched."""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_quantization_mean_amd import binding
    binding.load_library()
    return binding


def _t(shape, dtype):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def test_outputs_of_the_wrong_dtype_or_size(B):
    x = _t((64, 256), torch.bfloat16)
    with pytest.raises(TypeError):
        B.awq_act_stats(x, act_mean=_t(256, torch.float32))
    with pytest.raises(ValueError):
        B.awq_act_stats(x, act_mean=_t(255, torch.float64))
    with pytest.raises(ValueError):
        B.awq_act_stats(x, act_mean=_t((256, 2), torch.float64)[:, 0])  # strided
    act = _t(256, torch.float64)
    with pytest.raises(ValueError):
        B.awq_candidate_scales(act, 4, cand_scales=_t((3, 256), torch.float64))
    w = _t((32, 256), torch.bfloat16)
    with pytest.raises(ValueError):
        B.awq_quantize_pack(w, act, out={"codes": _t((32, 127), torch.uint8)})
    with pytest.raises(TypeError):
        B.awq_quantize_pack(w, act, out={"zeros": _t((32, 2), torch.float32)})
    with pytest.raises(TypeError):
        B.awq_search_scales(x, w, act, 4, out={"best_info": _t(2, torch.int64)})


def test_inputs_that_disagree(B):
    x = _t((64, 256), torch.bfloat16)
    act = _t(256, torch.float64)
    with pytest.raises(TypeError):  # the library takes one dtype for both operands
        B.awq_search_scales(x, _t((32, 256), torch.float32), act, 4)
    with pytest.raises(ValueError):
        B.awq_search_scales(x, [_t((32, 256), torch.bfloat16), _t((32, 384), torch.bfloat16)], act, 4)
    with pytest.raises(ValueError):
        B.awq_search_scales(x, _t((32, 384), torch.bfloat16), act, 4)
    with pytest.raises(TypeError):
        B.awq_search_scales(x, _t((32, 256), torch.bfloat16), _t(256, torch.float32), 4)
    with pytest.raises(ValueError):
        B.awq_quant_delta(_t((32, 256), torch.bfloat16), _t((4, 384), torch.float64))
    with pytest.raises(TypeError):
        B.awq_error_sse(x, _t((2, 32, 256), torch.float32))


def test_deployment_and_block_arguments(B):
    x = _t((8, 256), torch.bfloat16)
    codes = _t((16, 128), torch.uint8)
    steps = _t((16, 2), torch.int16)
    zeros = _t((16, 1), torch.uint8)
    with pytest.raises(ValueError):
        B.awq_w4a16_gemm(x, codes, steps, zeros, y=_t((8, 8), torch.float32))
    with pytest.raises(TypeError):
        B.awq_w4a16_gemm(x, codes, _t((16, 2), torch.int32), zeros)
    with pytest.raises(ValueError):
        B.awq_w4a16_gemm(x, _t((16, 64), torch.uint8), steps, zeros)
    with pytest.raises(TypeError):
        B.awq_export_fp16(_t((16, 2), torch.float32), _t((16, 2), torch.int32), out={"steps_f16": _t((16, 2),
                                                                                                    torch.int32)})
    with pytest.raises(TypeError):  # the block-level entry points take bfloat16 activations
        B.awq_mlp_hidden_ref(_t((8, 256), torch.float32), _t((64, 256), torch.bfloat16),
                             _t((64, 256), torch.bfloat16))
    with pytest.raises(ValueError):
        B.awq_mlp_hidden_ref(x, _t((64, 256), torch.bfloat16), _t((64, 128), torch.bfloat16))
    with pytest.raises(ValueError):
        B.awq_search_scales_mlp(x, _t((64, 256), torch.bfloat16), _t((64, 256), torch.bfloat16),
                                _t((32, 63), torch.bfloat16), _t(256, torch.float64))
