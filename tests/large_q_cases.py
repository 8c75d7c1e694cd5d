"""Layers with large rotations, shared by the GPU parity cases that check the
Cayley-Neumann adjoint (test_gpu_large_q.py) and the CPU test that shows
those cases can see every product of it (test_adjoint_sensitivity.py).

The workloads draw q ~ N(0, 1e-3^2), where the rotation is a few percent of
each output and the adjoint's terms in Q^2 and Q^3 sit far below the bfloat16
tolerance. Here sigma_q is raised so that ||Q||_2 (about 2 sigma_q sqrt(b) for
a random skew block) is about 0.45 ("mid") or 0.8 ("strong"). Only shapes and
draw parameters live here; no arithmetic.
"""

from orthogonal_equivalence_amd import synth


def _c(name, cfg_id, T, m, n, b, act, weight, sigma):
    return synth.LayerConfig(name, cfg_id, T, m, n, b, b, act, weight, sigma_q=sigma)


# (config, strength). T > m makes the bfloat16 backward fold H into the
# weight; T < m forms dY1 = dY2 H^T instead, so each block size meets both.
CASES = [
    # float32, general product engine for the CNP chain
    (_c("q_f32_b64_mid", 60, 200, 256, 320, 64, "f32", "f32", 0.03), "mid"),
    (_c("q_f32_b64_strong", 61, 300, 256, 320, 64, "f32", "f32", 0.055), "strong"),
    # bfloat16, fused block products (b a multiple of 128)
    (_c("q_bf16_b128_mid", 62, 300, 512, 640, 128, "bf16", "bf16", 0.02), "mid"),
    (_c("q_bf16_b128_strong", 63, 700, 512, 640, 128, "bf16", "bf16", 0.037), "strong"),
    (_c("q_bf16_b256_mid", 64, 1000, 768, 1024, 256, "bf16", "bf16", 0.015), "mid"),
    (_c("q_bf16_b256_strong", 65, 300, 768, 1024, 256, "bf16", "bf16", 0.026), "strong"),
    (_c("q_bf16_b512_mid", 66, 200, 1024, 1536, 512, "bf16", "bf16", 0.01), "mid"),
    (_c("q_bf16_b512_strong", 67, 1100, 1024, 1536, 512, "bf16", "bf16", 0.019), "strong"),
    # bfloat16, general product engine (block sizes 64 and 96, short last blocks)
    (_c("q_bf16_b64_strong", 68, 260, 448, 328, 64, "bf16", "bf16", 0.055), "strong"),
    (_c("q_bf16_b96_strong", 69, 200, 480, 600, 96, "bf16", "bf16", 0.043), "strong"),
    # int8 base weight, fused block products
    (_c("q_xq_b128_strong", 70, 400, 512, 768, 128, "bf16", "i8", 0.037), "strong"),
    # fp8 (E4M3) base weight, fused block products
    (_c("q_xf8_b128_strong", 71, 400, 512, 768, 128, "bf16", "f8", 0.037), "strong"),
]
