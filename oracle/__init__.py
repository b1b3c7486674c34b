"""CPU oracle of the decode-time KV-cache eviction step.

TEST INFRASTRUCTURE ONLY.  Plain, slow float64 numpy that states each step
of the method as the pages define it.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run anything in this package; the GPU library never does, and the
two share no code.

Sources (cited by page title and section):
  * BeaconKV — "长推理把显存吃爆了？BeaconKV：用几个「信标查询」预判模型会回头看什么"
    (sections: 观察 query 集 = 最近查询 + 信标查询; Continual FPS：有界内存的在线最远点采样;
    打分时的 RoPE 对齐; 📊 实验)
  * ReasonAlloc — "ReasonAlloc: Hierarchical Decoding-Time KV Cache ..." (Core Mechanism; Key Concepts)
  * EPIKV — "技术摘要：无需注意力矩阵的“顿悟感知型”KV 缓存驱逐策略"
    (方法论：EPIKV, parts 1 顿悟得分 and 3 时间趋势校正)

Parity status: every function below is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, library routines or invariants.
"""
from .kvevict_oracle import *  # noqa: F401,F403
