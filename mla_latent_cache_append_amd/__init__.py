"""libmla_absorb for AMD MI355X: weight-absorbed MLA decode over a paged bf16
latent cache. The C ABI is include/mla_absorb.h; ``native`` binds it with the
same names and ``step.DecodeStep`` strings the four calls into one decode step.
"""

from . import native  # noqa: F401
