"""CPU oracle (test infrastructure only; see smconv_oracle's header)."""
from .smconv_oracle import *  # noqa: F401,F403
from .smconv_oracle import (TAPS, CENTRE, DuplicateCoordinate, tap_offsets,  # noqa: F401
                            KERNEL_SIZES, taps_of, centre_of, mask_bit,
                            bf16_bits_to_f64, round_to_bf16, bf16_bits,
                            build_kernel_map, mask_sort, compact_pairs,
                            group_row_orders, tile_work, calibrate_order,
                            strided_out_shape, build_strided_map, strided_conv,
                            conv_accumulate, conv_rows, subm_conv, stage)
