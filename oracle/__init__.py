"""Plain, slow CPU oracle for low-bit KV-cache decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, helpers, tables or constant generators)
and imports nothing from ``dequant_decode_attention_amd``.

Every function follows a definition on one of three web pages and cites it
by page and section.  Page keys used throughout this repository:

* **[P1]** ihal.it/?p=61653 -- article on KV-cache quantization axes (KIVI,
  KVQuant, InnerQ).  It has no headings; it is cited by paragraph number and
  topic (e.g. "[P1 para 3, uniform integer quantization]").
* **[P2]** "VQKV: High-Fidelity and High-Ratio Cache Compression via
  Vector-Quantization", gist.science/it/paper/2603.16435, cited by section
  (e.g. "[P2 sec 2, key components: RSimVQ]").
* **[P3]** "Riepilogo Tecnico: RDKV - Allocazione dei Bit per
  Distorsione-Rate ...", gist.science/it/paper/2605.08317, cited by section
  title (the page numbers two sections "2.2": "bit-allocation pipeline" and
  "TriZone packed decoding").

Arithmetic conventions (each module's docstring states the readings it
takes where the pages leave a step open):

* fp16 inputs are widened to fp32 exactly; the quantizer runs in IEEE fp32
  with numpy float32 arrays (one rounding per operation, no fused
  multiply-add); ``np.rint`` rounds half to even; float32 -> float16 rounds
  to nearest even.
* attention is evaluated in fp64 over the dequantized values.

Parity status of each function is stated in its docstring; every function
here is pinned by tests in ``tests/test_oracle_*.py`` against closed forms,
brute force, library routines or invariants that the pages fix.
"""

from .quant import (
    GROUP,
    quantize_groups,
    quantize_k,
    quantize_v,
    dequantize_k,
    dequantize_v,
    pack_codes,
    unpack_codes,
    pack_v_codes,
    unpack_v_codes,
)
from .attention import (
    rope_frequencies,
    rope_rotate,
    attention_fp64,
    kivi_decode_attention,
)
from .zoned import (
    WIDTHS,
    zoned_layout,
    zoned_pack,
    zoned_decode_attention,
)
from .rvq import (
    rvq_encode,
    rvq_reconstruct,
    rvq_decode_attention,
    rvq_stage_distances,
)

__all__ = [
    "GROUP", "quantize_groups", "quantize_k", "quantize_v", "dequantize_k",
    "dequantize_v", "pack_codes", "unpack_codes", "pack_v_codes", "unpack_v_codes", "rope_frequencies",
    "rope_rotate", "attention_fp64", "kivi_decode_attention", "WIDTHS",
    "zoned_layout", "zoned_pack", "zoned_decode_attention", "rvq_encode",
    "rvq_reconstruct", "rvq_decode_attention", "rvq_stage_distances",
]
from .stream import (
    empty_stream,
    flush_count,
    kivi_append,
)
from .rdkv import (
    token_weights,
    token_weight_rows,
    channel_weights,
    widths_at,
    multiplier,
    allocate,
    budget_bits,
    rdkv_widths,
)
