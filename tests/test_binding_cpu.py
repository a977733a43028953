"""The Python binding checks what the C ABI cannot see -- element types,
element counts of outputs and scale buffers, and the device of every tensor --
and raises before any call reaches the library.  On a machine without a GPU
the tensors are host tensors: a wrong size or type is reported as such, and
right-sized host tensors are refused as not being on the GPU."""
import pytest
import torch

fq = pytest.importorskip("fp8_scaled_quantization_reduce_amd")


def f32(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


def bf16(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def u8(*shape):
    return torch.zeros(*shape, dtype=torch.uint8)


def i64(*shape):
    return torch.zeros(*shape, dtype=torch.int64)


X = bf16(256, 384)
N = X.numel()

BAD_CALLS = [
    # (call, exception, message fragment)
    (lambda: fq.fp8_amax(X, f32(2)), ValueError, "amax must have 1"),
    (lambda: fq.fp8_amax(u8(16), f32(1)), TypeError, "x must be"),
    (lambda: fq.fp8_quantize_tensor(X, 0, u8(N - 1), amax_in=f32(1)), ValueError, "q must have"),
    (lambda: fq.fp8_quantize_tensor(X, 0, f32(N), amax_in=f32(1)), TypeError, "q must be"),
    (lambda: fq.fp8_quantize_tensor(X, 0, u8(N), amax_in=f32(1), amax_out=f32(0)), ValueError, "amax_out"),
    (lambda: fq.fp8_quantize_tensor(X, 0, u8(N), scale_inv_in=torch.zeros(1, dtype=torch.float64)), TypeError,
     "scale_inv_in"),
    (lambda: fq.fp8_quantize_tensor_stats(X, 0, u8(N), i64(3), amax_in=f32(1)), ValueError, "stats"),
    (lambda: fq.fp8_quantize_tensor_stats(X, 0, u8(N), f32(4), amax_in=f32(1)), TypeError, "stats"),
    (lambda: fq.fp8_dequantize(u8(64), 0, f32(1), f32(63)), ValueError, "y must have"),
    (lambda: fq.fp8_dequantize(u8(64), 0, f32(1), bf16(64)), TypeError, "y must be"),
    (lambda: fq.fp8_quantize_rowwise_colwise(X, 0, q_row=u8(N), q_col=u8(N // 2), amax_in=f32(1)), ValueError,
     "q_col"),
    (lambda: fq.fp8_quantize_rowwise_colwise(bf16(N), 0, q_row=u8(N), amax_in=f32(1)), ValueError, "2-D"),
    (lambda: fq.fp8_quantize_block(X, 0, 128, u8(N), f32(5)), ValueError, "s_row must have 6"),
    (lambda: fq.fp8_quantize_block(X, 0, 1, u8(N), f32(256 * 3), u8(N), f32(384 * 1)), ValueError,
     "s_col must have 768"),
    (lambda: fq.fp8_quantize_block(X, 0, 128, u8(N), f32(6), u8(N), f32(5)), ValueError, "s_col must have 6"),
    (lambda: fq.fp8_quantize_mx(X, 0, u8(N), u8(256 * 11)), ValueError, "s_row must have 3072"),
    (lambda: fq.fp8_quantize_mx(X, 0, u8(N), f32(256 * 12)), TypeError, "s_row must be"),
    (lambda: fq.fp8_quantize_mx(X, 0, u8(N), u8(256 * 12), u8(N), u8(384 * 7)), ValueError, "s_col must have 3072"),
    (lambda: fq.fp8_update_scale_delayed(f32(16, 4), 0, f32(1), 0, 0, 0, 0, f32(3), f32(4)), ValueError,
     "scale must have 4"),
    (lambda: fq.fp8_update_scale_delayed(f32(16, 4), 0, f32(1), 0, 0, 0, 0, f32(4), f32(1)), ValueError,
     "scale_inv must have 4"),
    (lambda: fq.fp8_update_scale_delayed(f32(64), 0, f32(1), 0, 0, 0, 0, f32(1), f32(1)), ValueError, "hist"),
    (lambda: fq.fp8_quantize_delayed(X, 0, f32(16, 2), 0, 0, 0, 0, 0, f32(1), f32(2), u8(N)), ValueError,
     "scale must have 2"),
    (lambda: fq.fp8_quantize_delayed(X, 0, f32(16, 1), 0, 0, 0, 0, 0, f32(1), f32(1), u8(N - 16)), ValueError,
     "q must have"),
    (lambda: fq.fp8_scaled_gemm(u8(256, 512), 0, f32(1), u8(384, 512), 0, f32(1), fq.PER_TENSOR, bf16(256, 383)),
     ValueError, "shape mismatch"),
    (lambda: fq.fp8_scaled_gemm(u8(256, 512), 0, f32(2), u8(384, 512), 0, f32(1), fq.PER_TENSOR, bf16(256, 384)),
     ValueError, "sA must have 1"),
    (lambda: fq.fp8_scaled_gemm(u8(256, 512), 0, f32(256 * 4), u8(384, 512), 0, f32(2 * 4),
                                fq.BLOCK_1x128_128x128, bf16(256, 384)), ValueError, "sB must have at least 12"),
    (lambda: fq.fp8_scaled_gemm(u8(256, 512), 0, f32(256 * 4), u8(384, 512), 0, f32(3 * 4),
                                fq.BLOCK_1x128_1x128, f32(256, 384)), ValueError, "sB must have at least 1536"),
    (lambda: fq.fp8_scaled_gemm(u8(256, 512), 0, f32(256 * 16), u8(384, 512), 0, u8(384 * 16), fq.MXFP8,
                                bf16(256, 384)), TypeError, "sA must be"),
    (lambda: fq.fp8_scaled_gemm(u8(256, 512), 0, f32(1), u8(384, 512), 0, f32(1), fq.PER_TENSOR, u8(256, 384)),
     TypeError, "C must be"),
    (lambda: fq.fp8_scaled_gemm_fused(u8(256, 512), 0, f32(1), u8(384, 512), 0, f32(1), fq.PER_TENSOR,
                                      bf16(256, 384), bias=f32(383)), ValueError, "bias must have 384"),
    (lambda: fq.fp8_scaled_gemm_fused(u8(256, 512), 0, f32(1), u8(384, 512), 0, f32(1), fq.PER_TENSOR,
                                      u8(256, 384), out_fmt=fq.E4M3FN), ValueError, "c_scale_inv"),
    (lambda: fq.fp8_quantize_hybrid(X, 0, 1, 0, q_row=u8(N), q_col=u8(N + 1), amax_in=f32(1)), ValueError, "q_col"),
    (lambda: fq.fp8_quantize_hybrid_blockwise(X, fq.SUBQ_MXFP8, 0, fq.SUBQ_BLOCK_1x128, 1, q_row=u8(N),
                                              s_row=u8(3071), q_col=u8(N), s_col=f32(768)), ValueError,
     "s_row must have 3072"),
    (lambda: fq.fp8_quantize_hybrid_blockwise(X, fq.SUBQ_MXFP8, 0, fq.SUBQ_BLOCK_1x128, 1, q_row=u8(N),
                                              s_row=f32(3072), q_col=u8(N), s_col=f32(768)), TypeError,
     "s_row must be"),
    (lambda: fq.fp8_quantize_hybrid_blockwise(X, fq.SUBQ_MXFP8, 0, fq.SUBQ_BLOCK_1x128, 1, q_row=u8(N),
                                              s_row=u8(3072), q_col=u8(N), s_col=f32(767)), ValueError,
     "s_col must have 768"),
    (lambda: fq.fp8_quantize_hybrid_blockwise(X, fq.SUBQ_BLOCK_128x128, 0, fq.SUBQ_BLOCK_128x128, 1, q_row=u8(N),
                                              s_row=f32(6), q_col=u8(N - 1), s_col=f32(6)), ValueError, "q_col"),
    (lambda: fq.fp8_cast_stats(X, 0, f32(1), i64(5)), ValueError, "stats"),
    (lambda: fq.fp8_quantize_error_feedback(X, f32(N - 1), 0, f32(1), u8(N)), ValueError, "residual"),
    (lambda: fq.fp8_quantize_error_feedback(X, f32(N), 0, f32(1), u8(N), amax_out=f32(3)), ValueError, "amax_out"),
    (lambda: fq.fp8_quantize_tensor(X.t(), 0, u8(N), amax_in=f32(1)), ValueError, "contiguous"),
]


@pytest.mark.parametrize("i", range(len(BAD_CALLS)))
def test_binding_rejects_bad_buffers(i):
    call, exc, fragment = BAD_CALLS[i]
    with pytest.raises(exc, match=fragment):
        call()


GOOD_SHAPES_ON_HOST = [
    lambda: fq.fp8_amax(X, f32(1)),
    lambda: fq.fp8_quantize_tensor(X, 0, u8(N), amax_in=f32(1), scale_inv_out=f32(1)),
    lambda: fq.fp8_quantize_block(X, 0, 1, u8(N), f32(256 * 3), u8(N), f32(384 * 2)),
    lambda: fq.fp8_quantize_mx(X, 0, u8(N), u8(256 * 12), u8(N), u8(384 * 8)),
    lambda: fq.fp8_scaled_gemm(u8(256, 512), 0, f32(256 * 4), u8(384, 512), 0, f32(3 * 4),
                               fq.BLOCK_1x128_128x128, bf16(256, 384), amax_out=f32(1)),
    lambda: fq.fp8_scaled_gemm(u8(256, 512), 0, u8(256 * 16), u8(384, 512), 0, u8(384 * 16), fq.MXFP8,
                               f32(256, 384)),
    lambda: fq.fp8_quantize_error_feedback(X, f32(N), 0, f32(1), u8(N)),
    lambda: fq.fp8_quantize_hybrid_blockwise(X, fq.SUBQ_MXFP8, 0, fq.SUBQ_BLOCK_1x128, 1, q_row=u8(N),
                                             s_row=u8(3072), q_col=u8(N), s_col=f32(768)),
]


@pytest.mark.parametrize("i", range(len(GOOD_SHAPES_ON_HOST)))
def test_binding_refuses_host_tensors(i):
    """Every size and type is right; the tensors are not on the GPU."""
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        GOOD_SHAPES_ON_HOST[i]()
