"""The synthetic MoE-layer workloads (shapes, modes and input recipes).

They stand in for the serving workloads the pages measure (vLLM cells on
DeepSeek-V4 checkpoints), which need trained weights and datasets that are not
available: all inputs here are seeded and synthetic.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    K: int
    mode: str          # "w4a4_tensor" | "w4a4_token" | "w4a16" | "mxfp8" | "w4a4_token_4o6"
    #                    | "w4a4_token_mxfp4"
    act: str           # "swiglu" | "relu2"
    on_input: bool     # router weight applied before FC2 (input side)
    finalize: tuple    # finalize variants exercised: ("det",), ("fused",), ("det", "fused")
    logits: str        # make_logits kind
    seed: int = 0

    @property
    def N1(self) -> int:
        return 2 * self.I if self.act == "swiglu" else self.I

    @property
    def R(self) -> int:
        return self.T * self.K

    @property
    def wfmt(self) -> str:
        return {"mxfp8": "mxfp8", "w4a4_token_mxfp4": "mxfp4"}.get(self.mode, "nvfp4")


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_w4a4_tensor_T16_H256_I128_E8_K2", 16, 256, 128, 8, 2,
                 "w4a4_tensor", "swiglu", False, ("det",), "normal"),
        Workload("decode_w4a16_T256_H2048_I1024_E64_K6", 256, 2048, 1024, 64, 6,
                 "w4a16", "swiglu", False, ("det", "fused"), "uniform"),
        Workload("prefill_w4a4_token_T4096_H4096_I2048_E128_K8", 4096, 4096, 2048, 128, 8,
                 "w4a4_token", "swiglu", True, ("det", "fused"), "normal_bias"),
        # the same prefill layer under the 4-over-6 per-token activation contract
        Workload("prefill_w4a4_token4o6_T4096_H4096_I2048_E128_K8", 4096, 4096, 2048, 128, 8,
                 "w4a4_token_4o6", "swiglu", True, ("det", "fused"), "normal_bias"),
        # the same prefill layer with both GEMMs on NVFP4 operands re-blocked to
        # MXFP4 (the FP4 matrix cores; opt-in, adds a second rounding)
        Workload("prefill_w4a4_token_mxfp4_T4096_H4096_I2048_E128_K8", 4096, 4096, 2048, 128, 8,
                 "w4a4_token_mxfp4", "swiglu", True, ("det", "fused"), "normal_bias"),
        Workload("decode_w4a4_tensor_relu2_T64_H7168_I2048_E256_K8", 64, 7168, 2048, 256, 8,
                 "w4a4_tensor", "relu2", True, ("det",), "uniform"),
        Workload("prefill_mxfp8_zipf_T16384_H7168_I2048_E256_K8", 16384, 7168, 2048, 256, 8,
                 "mxfp8", "swiglu", False, ("fused",), "zipf"),
        # one GPU's share of the MXFP8 prefill under 8-way expert parallelism:
        # 32 local experts and an eighth of the routes (same mean group size)
        Workload("ep8_share_mxfp8_zipf_T2048_H7168_I2048_E32_K8", 2048, 7168, 2048, 32, 8,
                 "mxfp8", "swiglu", False, ("det", "fused"), "zipf"),
    ]
}

TINY = "tiny_w4a4_tensor_T16_H256_I128_E8_K2"
DECODE_W4A16 = "decode_w4a16_T256_H2048_I1024_E64_K6"
PREFILL_W4A4_TOKEN = "prefill_w4a4_token_T4096_H4096_I2048_E128_K8"
DECODE_W4A4_RELU2 = "decode_w4a4_tensor_relu2_T64_H7168_I2048_E256_K8"
PREFILL_MXFP8 = "prefill_mxfp8_zipf_T16384_H7168_I2048_E256_K8"
