"""CPU oracle of the Recurrent Looped Transformer decoder transition.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. It shares no code
with the GPU library; see ``rlt_oracle`` for the readings it fixes.
"""
from .rlt_oracle import (Config, Memory, Oracle, State, attend, behaviour_logprobs, build_memory,
                         importance_ratio, memory_entry, replay, retained_positions, ring_slot, rms_norm,
                         rope, rope_angles, sample, sigmoid, silu, state_from_ring,
                         state_to_ring, topk_order, trajectory_log_ratio, window_positions)
