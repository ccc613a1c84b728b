"""MI355X (gfx950) relative attention: HIP kernels behind a C ABI.

``prefill``, ``extend``, ``extend_mx``, ``decode``, ``decode_noalloc``,
``decode_paged``, ``decode_mx``, ``decode_plan``, ``prologue``,
``prologue_mx``, ``mx_quantize``, ``rel_logits``, ``backward`` and
``backward_plan`` call the compiled library ``librelattn.so``
(built in-tree by ``__graft_entry__.build()`` or
``python -m transformer_attention_query_amd.build``).  There is no fallback:
if the library is missing the calls raise.
"""

from .binding import (  # noqa: F401
    RelAttnError,
    backward,
    backward_plan,
    decode,
    decode_noalloc,
    decode_mx,
    decode_paged,
    decode_plan,
    extend,
    extend_mx,
    library_path,
    load_library,
    mx_quantize,
    prefill,
    prologue,
    prologue_mx,
    rel_logits,
    scale_factor,
    version,
)
