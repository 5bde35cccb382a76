"""Seeded synthetic input generation shared by the tests, the bench and the oracle checks."""
from .gen import (HEAD_DIM, WORKLOADS, BF16Tensor, Inputs, Workload, bf16_bits_to_f32,
                  custom_workload, f32_to_bf16_bits, make_inputs, norm_weights)
from .joint import JOINT_WORKLOADS, JointInputs, JointWorkload, make_joint_inputs, sequence_positions
from .block import BLOCK_WORKLOADS, BlockInputs, BlockWorkload, make_block_inputs

__all__ = ["HEAD_DIM", "WORKLOADS", "BF16Tensor", "Inputs", "Workload", "bf16_bits_to_f32",
           "custom_workload", "f32_to_bf16_bits", "make_inputs", "norm_weights", "JOINT_WORKLOADS", "JointInputs",
           "JointWorkload", "make_joint_inputs", "sequence_positions", "BLOCK_WORKLOADS", "BlockInputs",
           "BlockWorkload", "make_block_inputs"]
