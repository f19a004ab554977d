"""CPU oracle of the LatentMoE layer forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import, call, link or run anything in
this directory.  The GPU library never does; it shares no code with it.

Contents
  latentmoe_oracle.c  plain fp64 C implementation of the layer (per-token
                      forward, top-K' selection, gates, dispatch order)
  oracle.py           ctypes front end of the C file
  dense.py            numpy fp64 brute-force dense evaluation (every expert on
                      every token, masked), an independent formulation used
                      to pin the C file
  cost.py             closed-form parameter / byte / FLOP / combination counts

Pins (tests run with ``-m "not gpu"``): dense brute force vs C to 1e-12;
closed forms (identity weights give relu(x)^2; K' = N' gives the softmax
mixture; K' = 1 gives gate 1; zero router gives experts 0..K'-1 at 1/K';
standard MoE reduction at alpha 1 with identity projections); invariants
(gates sum to 1, distinct indices, dispatch is a bijection, degree-2
homogeneity of the routed and shared paths under fixed routing, token
permutation equivariance, expert relabelling invariance); every worked
number of the explainer page for ``cost.py``; and for FP8 (E4M3) expert banks
the format's defining values, all 256 byte values against torch's
float8_e4m3fn, equality with the bf16 path at power-of-two scales, and the
dense brute force with arbitrary per-column scales; for gated experts the
dense brute force with torch's silu and the exact odd/even identities of silu
under a sign flip of the gate banks; for the backward pass (orc_backward)
torch autograd on a dense formulation and central finite differences.  No
function here is left parity-unpinned.
"""
