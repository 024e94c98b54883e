"""Per-element error bound of the attention kernel's result against the exact
(float64) attention, from the kernel's arithmetic:

  S = scale Q K^T in fp32 (exact products of 16-bit values, fp32 sums of D
      terms): |dS| <= D u32 A_i with A_i = scale max_j sum_d |q_id k_jd|,
      which perturbs each P_ij by a relative 2 |dS| at most (the reference
      max moves too);
  P_ij = exp2 in fp32 against a reference max that may lag the row's true
      max by up to 2^8 (any reference gives the same quotient), then rounded
      to the input dtype (unit roundoff u_in); both the second product and
      the row sum l_i use the rounded values, so the normalised weights
      P_ij / l_i carry a relative 2 u_in at most;
  O = (sum_j P_ij V_j) / l_i accumulated in fp32 over Skv keys (the
      numerator and l_i: Skv u32 each, relative, first order);
  O rounded to the output dtype: u_out |O| <= u_out R_id.

Every term is a relative perturbation of a P_ij weighting |V_jd|, so

  |O_gpu - O| <= (3 u_in + u_out + 2 Skv u32 + 2 D u32 A_i) R_id + floor,

R_id = sum_j P_ij |V_jd|; the third u_in covers the exp2 argument and result
rounding (a few u32 each, relative) with room to spare; floor (1e-30) only
admits exact zeros.  u32 = 2^-24; u_in = u_out = 2^-11 (fp16) or 2^-8 (bf16)."""
import numpy as np

U32 = 2.0 ** -24
U16 = {0: 2.0 ** -11, 1: 2.0 ** -8}   # by dtype code: fp16, bf16


def tolerance(R, A, dtype, skv, dim):
    """Bound per element: R [rows, D], A [rows] (oracle.attention.attention_rows_weights)."""
    u = U16[dtype]
    rel = 3 * u + u + 2 * skv * U32 + 2 * dim * U32 * np.asarray(A)[:, None]
    return rel * R + 1e-30


def violations(got, want, R, A, dtype, skv, dim):
    """Boolean mask of elements outside the bound."""
    return np.abs(np.asarray(got, dtype=np.float64) - want) > tolerance(R, A, dtype, skv, dim)
