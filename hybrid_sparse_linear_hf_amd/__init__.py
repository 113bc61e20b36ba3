"""MI355X (gfx950) hybrid attention step of Hybrid Forcing.

The compute lives in libhf.so (HIP kernels behind the C ABI of include/hf.h);
`_lib` is its ctypes binding and `synth` draws seeded synthetic inputs.
"""

from ._lib import (HF_STEP_COMMIT, Geometry, HFError, Ring, abi_version, hf_block_select,  # noqa: F401
                   hf_block_select_hier, hf_cag_schedule,
                   hf_hybrid_step, hf_linear_absorb, hf_ring_append, hf_sparse_window_attn, new_workspace,
                   workspace_size, backward_workspace_size, new_backward_workspace, hf_sparse_window_attn_lse,
                   hf_hybrid_attn_backward, hf_linear_absorb_backward, Rope, hf_sparse_window_attn_rope,
                   hf_hybrid_step_rope, hf_hybrid_step_noalloc)
