"""libtwell: activation-sparse ReLU-gated FFN with TwELL-packed activations on MI355X (gfx950).

The compute lives in libtwell.so (hand-written HIP kernels behind a C ABI,
declared in include/twell.h); `twell` is its thin ctypes binding and
`autograd` a torch.autograd / nn.Module wrapper of the whole path.
"""
from . import twell  # noqa: F401
from .twell import (BF16, F32, TwellError, TwellFFN, alloc_hybrid, alloc_pack, alloc_workspace, ffn_bwd,  # noqa: F401
                    ffn_fwd, gate_pack, gate_pack_fp8, make_dims, n_tiles, pack_preact, quantize_e4m3, query_sizes,
                    route_hybrid)
