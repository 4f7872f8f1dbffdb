"""k-quant decode matvec for AMD MI355X (gfx950).

The compute path is the HIP library ``libkq.so`` (C ABI in ``include/kq.h``);
``_binding`` marshals arguments to it.  ``inputs`` generates the seeded
synthetic workloads.  Build the library with
``python -m quant_weight_matvec_amd.build``.
"""
from ._binding import (  # noqa: F401
    KQ_ERR_ALIAS, KQ_ERR_ALIGN, KQ_ERR_DEVICE, KQ_ERR_LAUNCH, KQ_ERR_NULL, KQ_ERR_SHAPE,
    KQ_ERR_UNSUPPORTED, KQ_MAX_K, KQ_MAX_M, KQ_MAX_TAIL_N, KQ_OK, KQ_QTYPE_Q4K, KQ_QTYPE_Q5K, KQ_QTYPE_Q6K,
    KQError, KQLibraryMissing, kq_build_info,
    kq_tune_small_m_plan, kq_tune_matvec_plan, kq_fused_residual_norm, kq_matmul_small_m, kq_matmul_small_m_noalloc, kq_ffn_gate_up_q4k_small_m,
    kq_matmul_small_m_workspace_bytes, KQ_SMALL_M_SCRATCH_BYTES,
    kq_matvec_q4k, kq_matvec_q5k, kq_embedding, kq_matvec_q6k, kq_matvec_group, kq_matvec_group_staged, KQ_MAX_GROUP, kq_ffn_gate_up_q4k, kq_probe_read_bw, kq_status_string, kq_tune_get_shape, kq_tune_set_shape, lib,
    kq_staged_bytes, kq_stage_activation, kq_matvec_staged, kq_ffn_gate_up_q4k_staged,
    kq_fused_residual_norm_staged, kq_ffn_tail_gate_up_q4k,
    kq_ffn_pass_q4k_q6k, kq_ffn_pass_workspace_bytes, kq_ffn_layer_table, KqFfnLayer,
    kq_tune_set_small_m_rows,
    kq_tune_set_gate_up_rows,
    KQ_MAX_FUSED_TAIL_K,
)
