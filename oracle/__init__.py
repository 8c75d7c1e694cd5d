"""Float64 CPU oracle for the POET-X reparameterized linear layer.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The HIP library and its Python binding never import, call or link it, and it
imports nothing from them: the two sides share only the seeded input
generator (``orthogonal_equivalence_amd.synth``), which holds none of the
method's arithmetic.

Every function is plain NumPy in float64 and follows the method as stated on
the zhichai.net digest of arXiv:2603.05500 ("POET-X: ... 单卡H100训练130亿参数
模型"), sections "1. 输入中心化架构" (input-centric evaluation),
"2. 块随机正交变换" (block-stochastic R = Psi^T Diag(G_1..G_ceil(m/b)) Psi) and
"3. Cayley-Neumann 参数化优化" (G = (I+Q)(I+Q+Q^2+Q^3), packed upper triangle).
"""

from .poetx_oracle import *  # noqa: F401,F403
