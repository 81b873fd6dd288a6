"""MI355X (gfx950) GPTQ-family layer-quantisation path: Python binding of libgptq_hip.so.

The entry points carry the C names of include/gptq.h:
    gptq_accumulate_hessian, gptq_prepare, gptq_asym_correction, gptq_quantize_layer (the layer path),
    gptq_prepare_groups, gptq_quantize_layer_groups (output-channel groups with a Hessian each, all groups per
    launch),
    gptq_act_order (act-order),
    gptq_device_status (the error latched on the device by a stream-ordered call), gptq_timer_enable /
    gptq_timer_read (per-class kernel times, a measurement aid),
    gptq_pack_codes, gptq_unpack_codes (storing the codes), gptq_hadamard_rotate (the rotation before it)
"""
from ._binding import (  # noqa: F401
    GPTQ_CALL_ACCUMULATE_HESSIAN, GPTQ_CALL_ACT_ORDER, GPTQ_CALL_ASYM_CORRECTION, GPTQ_CALL_PREPARE,
    GPTQ_CALL_QUANTIZE_LAYER,
    GPTQ_ERR_ARG, GPTQ_FLAG_CAE, GPTQ_FLAG_MSE, GPTQ_FLAG_SCALES_GIVEN, GPTQ_FLAG_STATIC_GROUPS, GPTQ_ERR_HIP, GPTQ_ERR_NONFINITE, GPTQ_ERR_NOT_PD, GPTQ_ERR_WORKSPACE, GPTQ_OK, LIB_PATH,
    GptqError, gptq_accumulate_hessian, gptq_act_order, gptq_asym_correction, gptq_hadamard_rotate, gptq_pack_codes, gptq_packed_words, gptq_prepare, gptq_prepare_groups,
    gptq_quantize_layer, gptq_quantize_layer_groups, gptq_unpack_codes, gptq_workspace_bytes, load, status_string, version,
    GPTQ_TIMER_CLASSES, gptq_device_status, gptq_gram_plan, gptq_timer_enable, gptq_timer_read,
)
