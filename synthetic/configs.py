"""The five synthetic layer configurations and their shape parameters.

Shapes follow the models the pages evaluate: OPT-6.7B / OPT-30B and a ReLU
Falcon-40B (KAIROX, Experimental setup), LLaMA2-7B ReGLU (PowerInfer, Method,
Insight 1; KAIROX, Experimental setup).  Predictor hidden sizes that the pages do
not give are d/4, which matches the two configurations that state one.
"""
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class FFNConfig:
    name: str
    d: int                 # model width (FFN input / output)
    f: int                 # FFN neurons
    h: int                 # predictor hidden width
    wdtype: str            # storage of FFN rows: 'f32' | 'f16' | 'bf16' | 'q4'
    act: str               # 'relu' | 'reglu'
    layers: int
    steps: int             # decode steps per layer in the workload
    batches: Tuple[int, ...]
    density: float         # mean per-token share of active neurons
    x_process: str         # 'iid' | 'ar1'
    planted: bool          # co-activated groups of 32 planted in the predictor
    tam: Optional[dict] = None
    workload: str = ""
    pred_q4: bool = False  # predictor W1 / W2 stored as int4 g32 (x stays fp16)
    pred_profile: str = "zipf"  # 'zipf': neuron i's predictor fires with probability p_i;
                                # 'iid': plain N(0, 1/fan_in) predictor, same rate for all

    @property
    def pdtype(self) -> str:
        """Storage of x and, unless pred_q4, of the predictor weights (q4 layers keep
        an fp16 x and, by default, an fp16 predictor)."""
        return "f16" if (self.wdtype == "q4" or self.pred_q4) else self.wdtype

    @property
    def pred_storage(self) -> str:
        """Storage of the predictor weights: 'q4' when pred_q4, else pdtype."""
        return "q4" if self.pred_q4 else self.pdtype

    @property
    def groups(self) -> int:
        return (self.f + 31) // 32


CONFIGS = {
    "C1": FFNConfig("C1", d=256, f=1024, h=64, wdtype="f32", act="relu", layers=1,
                    steps=8, batches=(1,), density=0.10, x_process="iid", planted=False,
                    pred_profile="iid", workload="tiny ReLU FFN d=256 f=1024 fp32"),
    "C2": FFNConfig("C2", d=4096, f=16384, h=1024, wdtype="f16", act="relu", layers=32,
                    steps=256, batches=(1,), density=0.08, x_process="ar1", planted=False,
                    workload="OPT-6.7B-shaped ReLU FFN d=4096 f=16384 h=1024 fp16, 32 layers"),
    "C3": FFNConfig("C3", d=4096, f=11008, h=1024, wdtype="bf16", act="reglu", layers=32,
                    steps=256, batches=(1, 4, 8), density=0.12, x_process="ar1", planted=True,
                    workload="LLaMA2-7B-shaped ReGLU FFN d=4096 f=11008 h=1024 bf16, 32 layers"),
    "C4": FFNConfig("C4", d=7168, f=28672, h=1536, wdtype="q4", act="relu", layers=48,
                    steps=256, batches=(1,), density=0.07, x_process="ar1", planted=False,
                    workload="OPT-30B-shaped ReLU FFN d=7168 f=28672 h=1536 int4-g32, 48 layers"),
    "C5": FFNConfig("C5", d=8192, f=32768, h=2048, wdtype="f16", act="relu", layers=60,
                    steps=512, batches=(1, 8, 32), density=0.06, x_process="ar1", planted=True,
                    tam={"lambdas": (0.8, 0.9, 0.95), "eps": 0.01, "K": 256},
                    workload="Falcon-40B-shaped ReLU FFN d=8192 f=32768 h=2048 fp16, 60 layers"),
}


def scaled(cfg: FFNConfig, **kw) -> FFNConfig:
    """A copy of `cfg` with some fields replaced (smaller test shapes keep the
    generator recipe of the full configuration)."""
    name = kw.pop("name", cfg.name + "s")
    return replace(cfg, name=name, **kw)
