"""Python binding of libdqip.so: the dynamic quantized inner product,
QuantizeLinear / DequantizeLinear, the requantizing 1x1 QLinearConv, the
quantized matrix products, the element-wise quantized operators, the
general QLinearConv and DynamicQuantizeLSTM on AMD Instinct MI355X (gfx950).

Argument marshalling only: every step runs in the library's HIP kernels.
The functions carry the names of the C entry points declared in
``include/dqip.h``; tensors are torch tensors on the GPU (their data pointers
are passed), ``stream`` defaults to torch's current stream. A missing library
raises: there is no fallback.
"""
from ._binding import (  # noqa: F401
    DQ_ACT_IDENTITY, DQ_ACT_LEAKY_RELU, DQ_ACT_RELU, DQ_BF16, DQ_ERR_ALLOC, DQ_ERR_ARG, DQ_F16,
    DQ_ERR_HIP, DQ_ERR_RANGE, DQ_ERR_STATE, DQ_ERR_TYPE, DQ_F32, DQ_I8, DQ_K_MAX, DQ_OK,
    DQ_PER_TENSOR, DQ_U8, DQError, LIB_PATH, dqip_enabled, dqip_external_buffer_size,
    dqip_forward, dqip_forward_accumulators, dqip_info, dqip_init, dqip_internal_buffer_size,
    dqip_last_error, dqip_profile_begin, dqip_profile_end, dqip_read_quantized_a, dqip_read_quantized_b, dqip_release,
    dqip_set_params, exported_symbols, load, qlinear_conv1x1, qlinear_dequantize, qlinear_quantize,
    DQ_QGEMM_K_MAX, DQ_QGEMM_BATCH_MAX, DQ_QGEMM_BATCH_RANK_MAX, dq_qgemm_init_batched,
    dq_qgemm_forward, dq_qgemm_forward_accumulators, dq_qgemm_info, dq_qgemm_init,
    dq_qgemm_release, dq_qgemm_set_b, dq_mul_integer, dq_reduce_sum_integer, qlinear_add,
    qlinear_concat, qlinear_leaky_relu, qlinear_mul, qlinear_reduce_mean, qlinear_sigmoid,
    qlinear_dequantize_f16, qlinear_quantize_f16, dq_qconv_forward, dq_qconv_info,
    dq_qconv_init, dq_qconv_output_shape, dq_qconv_release, dq_qconv_set_w,
    DQ_LSTM_BIDIRECTIONAL, DQ_LSTM_FORWARD, DQ_LSTM_HIDDEN_MAX, DQ_LSTM_REVERSE, RNN_ACTIVATIONS,
    dq_lstm_forward, dq_lstm_info, dq_lstm_init, dq_lstm_release, dq_lstm_set_weights,
    lstm_activation_slots, dq_probe_copy, dq_probe_mfma_loop, dqip_forward_noalloc,
    DQIP_NOALLOC_SCRATCH_BYTES,
)
