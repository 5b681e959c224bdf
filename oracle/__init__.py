"""Plain CPU oracle of the routed mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The GPU library never routes through it, and it shares no code with
the GPU library (no kernels, headers, helpers, tables or constants): it reads
plain NumPy arrays and returns plain NumPy arrays.

What it computes is the layer described on the page "Optimising Ling-2.6-1T on
TPU with SGLang-JAX: hiding MoE data movement behind compute with one Pallas
kernel" (cited below as *Ling-2.6-1T on TPU*): routing to the top-k experts,
per-token fp8 activation quantisation before the scatter, a gated expert FFN
(W1/W3 gate-up projection, SiLU times gate, W2 down projection) on per-channel
fp8 weights with scales applied after the full reduction, an optional shared
expert, and the weighted gather back into token order.  The MXFP4 weight
format and the LatentMoE expert shape with its RMSNorm come from the page
"Feasibility of porting Kimi K3 to the Google TPU ecosystem" (cited as
*Kimi K3 on TPU*) and the page "Implementation gaps: advanced optimisations"
of the sglang-jax reference wiki (cited as *sglang-jax gap list*).

Everything is float64 except at the rounding points the method itself
defines (the fp8 e4m3 quantisation of the activations before the scatter,
the bf16 intermediate h, and the final bf16 output).

Pins (each checked in ``tests/test_oracle_*.py`` against something other than
the oracle itself): codecs against the OCP definitions and against torch's
float8/bfloat16 casts; routing against brute force, textbook softmax and tie
cases; permutation against NumPy's stable argsort; the FFN against a dense
gated FFN (one expert, top-1), token-permutation invariance, zero routing
weights, power-of-two linearity, a per-token brute-force loop, hand-computed
closed-form examples and an MXFP4 / fp8 cross-check; the FLOP and byte
accounting against the worked figures the pages print; the LatentMoE block
(``latent``: MXFP4 down/up projections around the routed core, bf16 shared
experts on the hidden stream, *Kimi K3 on TPU* §2.4-2.5) against exact
products of representable weights, selection-matrix wiring through the
pinned core, a closed form of the shared path, torch's float64 linear and
exact power-of-two scalings; per-block fp8 weights (``fmt="fp8_block"``, one
scale per 128 x 128 tile, *Ling-2.6-1T on TPU* §5) against a hand-worked
closed form, the per-channel special case and a brute-force loop.  The numerical MoE
output as a whole is otherwise "parity unpinned": the pages print no worked
example of it.
"""

from . import codecs, moe, accounting, latent  # noqa: F401
from .moe import (  # noqa: F401
    route,
    quantize_tokens,
    expert_counts_offsets,
    permute_rows,
    expert_ffn,
    combine,
    forward,
)
