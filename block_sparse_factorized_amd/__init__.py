"""Block-sparse causal factorized self-attention (Sparse Transformer strided
and fixed patterns) for AMD Instinct MI355X (gfx950).

The compute path is libsa.so (C ABI in include/sa.h, HIP kernels in csrc/);
this package is a thin ctypes binding with the same names.  Importing it
fails if the library has not been built.
"""
from ._binding import (  # noqa: F401
    EXPORTED,
    FWD_FORMS,
    LIB_PATH,
    PATTERNS,
    SA_BF16,
    SA_ERR_ALLOC,
    SA_ERR_HIP,
    SA_ERR_INVALID_ARG,
    SA_ERR_UNSUPPORTED,
    SA_F32,
    SA_OK,
    Layout,
    SAError,
    library,
    sa_bwd,
    sa_bwd_dkdv,
    sa_bwd_dq,
    sa_bwd_dq_rowterms,
    sa_bwd_noalloc,
    sa_bwd_rowterms,
    sa_bwd_workspace_size,
    sa_fwd,
    sa_layout_build,
    sa_layout_destroy,
    sa_layout_export,
    sa_layout_info,
    sa_layout_set_compact_view,
    sa_layout_set_residue_view,
    sa_layout_view_info,
    sa_set_fwd_form,
    sa_set_one_paths,
    sa_set_split,
    sparse_attention,
)
