"""Work counts of the three kernels, per output pair and direction (bytes and
flops that the algorithm must move / execute; used for roofline fractions).

Per pair (b, i, j), storage element size `esz` (2 for bf16, 4 for fp32):
  k1 input gate   reads z (c_z) and the mask (1), writes a and b (2c)
                  flops: four c_z -> c projections = 8 c c_z
  k2 contraction  reads a and b rows once (2c), writes x (c)
                  flops: 2 N c
  k3 output gate  reads x (c), z (c_z), mask (1); writes out (c_z)
                  flops: c -> c_z projection 2 c c_z, c_z -> c_z gate 2 c_z^2
and of the pair transition (one kernel), per pair:
  pair_transition reads z (c_z) and the mask (1), writes out (c_z)
                  flops: c_z -> hidden and hidden -> c_z linears, 4 c_z hidden
"""

MI355X_PEAK = {
    "hbm_GBps": 8000.0,           # HBM3E
    "bf16_TFLOPs": 2516.6,        # dense MFMA
    "fp32_mfma_TFLOPs": 157.3,
}


def kernel_work(n, c_z, c, esz):
    return {
        "k1_input_gate": {"bytes": esz * (c_z + 1 + 2 * c), "flops": 8 * c * c_z},
        "k2_contract": {"bytes": esz * 3 * c, "flops": 2 * n * c},
        "k3_output_gate": {"bytes": esz * (c + c_z + 1 + c_z), "flops": 2 * c * c_z + 2 * c_z * c_z},
    }


def flops_per_pair(n, c_z, c):
    """Matmul flops of one direction per output pair: 2Nc + 10 c c_z + 2 c_z^2."""
    return 2 * n * c + 10 * c * c_z + 2 * c_z * c_z


def transition_work(c_z, hidden, esz):
    return {"bytes": esz * (2 * c_z + 1), "flops": 4 * c_z * hidden}
