"""CPU oracle (test infrastructure only; see sbn_oracle's header)."""

from .sbn_oracle import *  # noqa: F401,F403
from .sbn_oracle import (  # noqa: F401
    absmean_gamma, act_absmax, act_scale, bf16_to_f32, bitlinear_forward,
    boundary_elements_act, boundary_elements_weight, check_pattern, combinatorial_metadata_bits,
    compact_pack, compact_row_bytes, compact_unpack, mask_rank, mask_unrank, rank_bits,
    rank_pack, rank_row_bytes, rank_unpack, forward_with_outliers, outlier_matrix,
    outlier_select, pack_with_outliers,
    dequantize, f32_to_bf16_rne, int_matmul, layernorm_bf16, layernorm_quantize_act,
    mask_flips, nm_keep_mask, pack_nm_ternary, quantize_act, rpf_pack,
    rpf_row_bytes, rpf_unpack, ste_dx, ste_dx_abs, ternary_codes, variance_correction,
)
