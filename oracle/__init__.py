"""Float64 CPU oracle for selector-driven block-sparse landmark attention.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU-baseline leg
of the benchmark may import anything from this package.  The product path (the HIP
library and its Python binding) never imports it, and this package imports nothing
from the product path.

Pages cited (their titles, translated from Russian; the original title follows):

* SAS page -- "Scientists taught transformers to select context directly rather than
  by imitating full attention" (iitog.ru; "Учёные научили трансформеры отбирать
  контекст напрямую, а не через имитацию полного внимания").
* HiLS page -- "HiLS-Attention: hierarchical sparse attention for ultra-long context in
  language models" (iitog.ru; "HiLS-Attention: иерархическое разреженное внимание для
  сверхдлинного контекста в языковых моделях").
* LSA page -- "Latent Sparse Attention" (rit.work blog, "latent-sparse-attention-ultra-
  long-context"); its first section is "The index stops scanning the whole context"
  ("Индекс перестаёт перебирать весь контекст").

Every function is pinned by a test in tests/test_oracle.py against something other than
itself (a library routine, a closed form, an invariant, or brute force on tiny inputs).
"""

from .bsa_oracle import (  # noqa: F401
    round_to_dtype,
    landmarks,
    selector_vectors,
    decode_selector_vectors,
    block_scores,
    select_row,
    select_all,
    log_sigmoid,
    sas_gates,
    attend_rows,
    hils_chunks,
    attend_hils_rows,
    prefill,
    prefill_rows,
    decode,
    n_blocks,
    gather_pages,
    decode_paged,
    attend_rows_grad,
    sas_gates_grad,
    hils_rows_grad,
    prefill_backward,
    ward_clusters,
    lsa_index,
    lsa_select_row,
    lsa_tree_centres,
    lsa_tree_select_row,
    update_landmarks,
    update_landmarks_paged,
    lsa_update_index,
)
