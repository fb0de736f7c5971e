"""Plain, slow, fp64 CPU definition of the on-the-fly SO(2) equivariant graph
attention forward pass.

TEST INFRASTRUCTURE ONLY.  This package is the oracle that the HIP path is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
the HIP library (``so_equivariant_graph_amd``) and never imports it; the
HIP library never imports this package.

What it follows (page titles as printed on the source pages):

* "E2Former-V2: On-the-Fly Equivariant Attention with Linear Activation
  Memory", technical summary, section 2.1 (EAAS: rotate each edge into the
  frame aligned with the edge vector, where the spherical harmonics of the
  edge keep only m = 0, and replace the dense SO(3) contraction by sparse
  block-wise linear maps) and section 2.2 (node-centric attention: query and
  key are SO(3)-invariant scalar projections, geometry enters only through
  the values, a softmax over the neighbours N(i) within the cutoff).
* "EquiformerV3: Scaling Efficient, Expressive, and General
  SE(3)-Equivariant Graph Attention Transformers", technical summary,
  section 2.B.3 (smooth radius cutoff: the envelope sits inside attention,
  denominator included).
* "DPA4: Pushing the Accuracy-Cost Frontier of Interatomic Potentials with
  EMFA SO(2) Convolution", technical summary, section 2.1 A3
  (envelope-gated attention, weights from the invariant l = 0 section).

The pages print no equations, so every formula here is a stated reading
(each module says which, and why).  Parity status of every
function is pinned by ``tests/test_oracle_*.py`` against closed forms,
invariants and brute force; the absolute output values of the layer are not
printed on the pages (no worked example exists), so the layer as a whole is
pinned by symmetry, special cases and a hand-worked two-atom case.

Modules
-------
sh         real spherical harmonics (no Condon-Shortley phase, z polar)
wigner     Wigner-D blocks by exact quadrature, edge-frame rotation
neighbors  brute-force O(N^2) radius graph in fp64, CSR output
attention  the per-edge loop: rotate, gate, SO(2) map, rotate back,
           two-pass softmax with the envelope, aggregate
attention_grad  gradients of the layer (node features, positions, every
           weight) by autograd through a PyTorch fp64 copy of the forward,
           pinned to finite differences of the numpy forward
norm       the merged RMS layer norm of the node features ("EquiformerV3"
           technical summary, section 2.B.1)
swiglu     the SwiGLU-S2 activation of the node features ("EquiformerV3"
           technical summary, section 2.C)
"""

from .sh import real_sh, n_comp
from .wigner import wigner_d_blocks, frame_rotation, rot_z
from .neighbors import neighbors_bruteforce
from .attention import (
    so2_attention_ref,
    envelope,
    radial_gaussians,
    unpack_so2,
    so2_weight_count,
    max_rel_error,
)
from .attention_grad import so2_attention_grad_ref
from .norm import merged_rms_norm_ref
from .swiglu import s2_grid, swiglu_s2_ref

__all__ = [
    "real_sh",
    "n_comp",
    "wigner_d_blocks",
    "frame_rotation",
    "rot_z",
    "neighbors_bruteforce",
    "so2_attention_ref",
    "so2_attention_grad_ref",
    "merged_rms_norm_ref",
    "swiglu_s2_ref",
    "s2_grid",
    "envelope",
    "radial_gaussians",
    "unpack_so2",
    "so2_weight_count",
    "max_rel_error",
]
