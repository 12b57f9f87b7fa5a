"""fp64 CPU oracle (test infrastructure only; see ``oracle/attention.py``)."""

from .attention import (  # noqa: F401
    kv_page_update,
    gather_kv,
    paged_attention,
    paged_attention_rows,
    varlen_attention,
    split_bounds,
    split_partial,
    fold,
    split_fold_attention,
)
from .rmsnorm import rmsnorm  # noqa: F401,E402
from .gemm import gemm  # noqa: F401,E402
