"""fp64 CPU oracle of the parallel DiT block (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP path.
"""
from .dit_block import (  # noqa: F401
    FLAG_NO_GATE, FLAG_NO_RESIDUAL, adaln_ref, attention_ref, block_ref, head_rms_norm,
    layer_norm, rel_l2, rope4_ref, rope_omega, silu, softmax_rows, stream_index, swiglu_ref,
    widen_bf16)
from .stack import cfg_combine, round_bf16, stack_branch, stack_cfg_ref  # noqa: F401
from .sampler import (  # noqa: F401
    denoise_step, euler_cfg_step, flow_sigmas, linear, modulation, output_layers, sample,
    sampler_prepare, time_embedding, timestep_sinusoid)
from .fp8 import (  # noqa: F401
    block_ref_fp8, dequantize_rows, e4m3_decode, e4m3_round, e4m3_values, fp8_linear,
    quantize_rows)
