"""Plain fp64 CPU oracle for absorbed Multi-head Latent Attention decode.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(``mla_latent_cache_append_amd``, the HIP kernels and the C ABI) never imports,
links or calls anything here, and this package imports nothing from it.

Sources (cited by title and section throughout):

* [AUDIT]  llm-atlas page "DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界"
           (research/DEEPSEEK_MLA_ABSORB_AUDIT.md)
* [MLA80]  CSDN page "80 行 PyTorch 从零写 DeepSeek 的 MLA：量一遍 KV cache、踩一遍
           absorption ..."
* [TRACE]  llm-atlas page "DeepSeek-V2-Lite 真实权重执行审计"
           (research/DEEPSEEK_V2_LITE_TRACE.md)

Every function in :mod:`oracle.mla` is pinned by ``tests/test_oracle_*.py``
against facts the pages or mathematics fix (printed byte counts, the
absorption identity, a library SDPA, brute force, closed forms), and the
input decoder ``bf16_bits_to_f64`` against torch's bfloat16 -> float64
conversion on all 65,536 bit patterns (``tests/test_oracle_decode_inputs.py``,
with a planted binary16 misreading it must catch). The
real-weight error tables of [AUDIT] §5 are the only page figures this oracle
cannot reproduce (the checkpoint and prompt are not available), and nothing
here claims to.
"""

from . import mla  # noqa: F401
