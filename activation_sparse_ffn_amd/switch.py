"""Choice between the sparse step and the dense FFN for a batch (PowerInfer page,
Implementation: long inputs go to dense GPU computation in the prefill stage;
KAIROX page, Future work: choose sparse or dense kernels online from the batch).

The sparse step reads the predictor and the rows of the union of the batch's
masks; the dense FFN reads every row and no predictor.  With calibration
frequencies p_i (share of calibration tokens whose mask holds neuron i) and
tokens taken as independent, the expected union of B tokens is
sum_i 1 - (1 - p_i)^B.  Each path's time is its bytes over the bandwidth that path
reaches on the device, measured (e.g. by the benchmark at a few batch sizes); the
switch takes the faster one.
"""
from dataclasses import dataclass

import numpy as np


def expected_union(p: np.ndarray, B: int) -> float:
    """Expected number of neurons active for at least one of B independent tokens."""
    p = np.asarray(p, dtype=np.float64)
    return float(np.sum(1.0 - np.power(1.0 - p, B)))


@dataclass
class SparseDenseSwitch:
    """pred_bytes: predictor weights read per step; row_bytes: bytes of one neuron's
    rows (up, gate, bias, down); f: neurons; sparse_gbps / dense_gbps: bandwidth each
    path reaches (measured)."""
    pred_bytes: float
    row_bytes: float
    f: int
    sparse_gbps: float
    dense_gbps: float

    def sparse_us(self, k: float) -> float:
        return (self.pred_bytes + k * self.row_bytes) / (self.sparse_gbps * 1e3)

    def dense_us(self) -> float:
        return self.f * self.row_bytes / (self.dense_gbps * 1e3)

    def use_dense(self, k: float) -> bool:
        """Dense when it is faster for an expected union of k neurons."""
        return self.dense_us() < self.sparse_us(k)

    def crossover_k(self) -> float:
        """Union size above which the dense FFN is faster (may exceed f: never)."""
        return (self.dense_us() * self.sparse_gbps * 1e3 - self.pred_bytes) / self.row_bytes

    def choose(self, p: np.ndarray, B: int) -> str:
        return "dense" if self.use_dense(expected_union(p, B)) else "sparse"
