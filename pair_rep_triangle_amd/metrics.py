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
and of triangular attention (H heads of width d, per pair and node):
  ka_project      reads z (c_z) and the mask (1); writes q, k, gate, v (4 H d) in the
                  storage type, the pair bias (H) and the mask (1)
                  flops: LayerNorm'd z times 4 H d + H projection rows, 2 c_z (4 H d + H)
  ka_core         reads q, gate, k, v (4 H d; k and v of a row once) and the mask (1),
                  the pair bias once per item (H); writes out (c_z)
                  flops: q.k and p.v over N keys per head, 4 N H d, plus the output
                  projection 2 H d c_z; one exponential per (query, key, head): N H
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


def attention_work(n, c_z, heads, d, esz):
    """Per pair. ka_project reads z and the mask and writes q, k, gate, v, the per-head
    bias and one key-valid bit; ka_core reads all of those once and writes out."""
    hd = heads * d
    return {
        "ka_project": {"bytes": esz * (c_z + 1 + 4 * hd + heads) + 0.125,
                       "flops": 2 * c_z * (4 * hd + heads)},
        "ka_core": {"bytes": esz * (4 * hd + heads + c_z) + 0.125,
                    "flops": 4 * n * hd + 2 * hd * c_z, "exps": n * heads},
    }


# transcendental rate of the chip: 256 CUs x 4 SIMDs, each 8 v_exp_f32 results per cycle
# (half the 16-lane rate of plain fp32 VALU; CDNA 4 doubled the transcendental rate), at
# the 2.4 GHz peak engine clock. A one-SIMD probe measured 5.4 ns per 64-lane exp2 at about
# 2.0 GHz (1.2e13/s over the chip), above what a quarter rate would allow.
MI355X_EXP_PER_S = 256 * 4 * 8 * 2.4e9
