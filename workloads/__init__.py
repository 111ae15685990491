"""Seeded synthetic inputs for the preallocated-KV-cache GQA path.

This package is shared by the tests, the benchmark and the CPU oracle. It
holds random draws, the float32 -> bfloat16 storage rounding of those draws,
workload shapes and call schedules (which row receives how many tokens in which
call). It holds none of the method's arithmetic: no cache writes, no masks,
no softmax.
"""

from .synth import (  # noqa: F401
    Shape,
    TINY_FP32,
    LLAMA8B_DECODE,
    LLAMA8B_VERIFY,
    LLAMA8B_CHUNKED_PREFILL,
    LLAMA8B_RAGGED,
    LLAMA8B_WINDOW_DECODE,
    llama8b_decode_shard,
    WORKLOADS,
    to_bf16_bits,
    bf16_bits_to_f32,
    storage_np_dtype,
    draw,
    prefix_kv,
    step_inputs,
    schedule_to_lengths,
    tiny_schedule,
    trial_spec,
    ragged_rows,
    ring_schedule,
)
