"""libqwattn: the Qwen3 attention-sublayer core (QK-Norm, rotate-half RoPE,
causal grouped-query attention) as hand-written HIP kernels for MI355X (gfx950)
behind a C ABI.  ``inputs`` and ``accounting`` are importable without the
library; the compute entry points load it on first use and raise if it is not
built."""

from . import accounting, inputs  # noqa: F401
