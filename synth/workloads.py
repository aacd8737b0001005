"""The synthetic workloads: shapes, sizes, value distributions and seeds of the
five configurations the step is tested and measured on.  Holds none of the
step's arithmetic.

Recipe (all values seeded; element j of every tensor is a function of its
stream key and its GLOBAL flat index j, so per-rank slices, full buffers and
sampled elements agree):
  gradient of rank k at step s   sigma_g * z(key("grad", name, s, k), j)
  pre-reduced gradient at step s sigma_g * z(key("grad", name, s, "reduced"), j)
  fp32 master at step 0          0.02 * z(key("master", name), j)
  m = v = 0 at step 0; flat padding elements (j >= T) are 0 everywhere.
z is the Irwin-Hall(12) standard variate of synth_cpu.c / synth_gpu.hip
(bounded at +-6); values are rounded to the storage format.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

F32, F16, BF16 = 0, 1, 2
SUM, AVG = 0, 1

TINY_MLP = (512 * 1024, 1024, 1024 * 512, 512)                         # 1,050,112
LLAMA7B_BLOCK = (4096 * 4096,) * 4 + (11008 * 4096, 11008 * 4096, 4096 * 11008, 4096, 4096)

HP = dict(lr=3e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=1.0)


@dataclass(frozen=True)
class Workload:
    name: str
    numels: Tuple[int, ...]
    n_ranks: int
    rank: int
    grad_dtype: int            # storage format of the gradients
    param_dtype: int           # format of the All-Gather slot
    reduce: bool               # True: N raw rank buffers; False: one pre-reduced shard
    op: int = AVG
    loss_scale: float = 65536.0
    dynamic: bool = False
    window: int = 1000
    steps: int = 3
    quant_block: int = 0       # 0: no INT8 payload
    grad_sigma: float = 1e-3
    master_sigma: float = 0.02
    full_allgather: bool = True  # False: the slot is its own buffer (offset 0)
    inject: Optional[Tuple[int, int, int, float]] = None  # (step, rank buffer, flat index, value)
    micro_steps: int = 1       # > 1: gradient accumulation over this many micro-steps
    grad_int8: bool = False    # rank gradients arrive INT8-quantised (blocks of 256)
    hp: dict = field(default_factory=lambda: dict(HP))

    @property
    def total(self):
        return sum(self.numels)

    @property
    def shard(self):
        return -(-self.total // self.n_ranks)

    @property
    def padded(self):
        return self.shard * self.n_ranks

    @property
    def start(self):
        return self.rank * self.shard


WORKLOADS = {
    # 2-layer MLP FlatParameter over 4 simulated ranks, rank 0, fp16 grads,
    # static scale 65536, clip 1.0, AVG, 3 steps
    "tiny_mlp_n4": Workload("tiny_mlp_n4", TINY_MLP, 4, 0, F16, F16, True, steps=3),
    # 1.5B GPT-like flat parameter over 64 ranks, rank 0; 64 fp16 rank
    # buffers reduced with AVG; dynamic scale from 2^16, window 1000; 10 steps
    "gpt1p5b_n64": Workload("gpt1p5b_n64", (1_500_000_000,), 64, 0, F16, F16, True,
                            dynamic=True, steps=10),
    # 10B over 8 ranks, rank 7 (slot offset 8.75e9); pre-reduced fp16 shard;
    # static 2^16; fp16 write-back into the full 20 GB All-Gather buffer; 5 steps
    "10b_n8": Workload("10b_n8", (10_000_000_000,), 8, 7, F16, F16, False, steps=5),
    # the same shard with the 8 raw fp16 rank buffers reduced (AVG) in the step
    "10b_n8_reduce8": Workload("10b_n8_reduce8", (10_000_000_000,), 8, 7, F16, F16, True,
                               steps=5),
    # one Llama-style 7B block over 8 ranks, rank 3; 8 bf16 buffers; dynamic
    # scale from 2^16; step 2 injects +inf in buffer 5 inside rank 3's slice
    "llama7b_block_n8": Workload("llama7b_block_n8", LLAMA7B_BLOCK, 8, 3, BF16, BF16, True,
                                 dynamic=True, steps=3,
                                 inject=(1, 5, 75_893_760 + 12_648_960, float("inf"))),
    # 70B over 64 ranks, rank 63; pre-reduced bf16 shard, scale 1; clip 1.0
    # (active); bf16 write-back plus INT8 blocks of 256; slot-sized buffers
    "70b_n64_int8": Workload("70b_n64_int8", (70_000_000_000,), 64, 63, BF16, BF16, False,
                             loss_scale=1.0, steps=5, quant_block=256, full_allgather=False),
    # gradient accumulation (2kiu.com §5.1: gradient_accumulation_steps 2):
    # each step reduces 2 micro-steps' rank buffers into the fp32 shard
    "tiny_mlp_n4_accum2": Workload("tiny_mlp_n4_accum2", TINY_MLP, 4, 1, F16, F16, True,
                                   steps=3, micro_steps=2),
    "10b_n8_accum2": Workload("10b_n8_accum2", (10_000_000_000,), 8, 7, F16, F16, True,
                              steps=5, micro_steps=2),
    # quantised gradient Reduce-Scatter ("DeepSpeed 与 FSDP", ZeRO++): every rank's
    # fp16 slice quantised to INT8 + block scales before the reduce
    "tiny_mlp_n4_qg": Workload("tiny_mlp_n4_qg", TINY_MLP, 4, 2, F16, F16, True, steps=3,
                               grad_int8=True),
    "gpt1p5b_n64_qg": Workload("gpt1p5b_n64_qg", (1_500_000_000,), 64, 0, F16, F16, True,
                               dynamic=True, steps=10, grad_int8=True),
    "10b_n8_qg": Workload("10b_n8_qg", (10_000_000_000,), 8, 7, F16, F16, True, steps=5,
                          grad_int8=True),
}


@dataclass(frozen=True)
class Gather:
    """The receiving side of an INT8 All-Gather: n_ranks slots of the flat
    parameter's codes and block scales, dequantised into the full flat buffer."""
    name: str
    numels: Tuple[int, ...]
    n_ranks: int
    out_dtype: int
    block: int = 256
    scale_sigma: float = 4.7e-4   # ~ amax/127 of an N(0, 0.02) block

    @property
    def total(self):
        return sum(self.numels)

    @property
    def shard(self):
        return -(-self.total // self.n_ranks)

    @property
    def padded(self):
        return self.shard * self.n_ranks

    @property
    def n_blocks(self):
        return -(-self.shard // self.block)


GATHERS = {
    "tiny_mlp_n4_gather": Gather("tiny_mlp_n4_gather", TINY_MLP, 4, F16),
    # one FSDP unit: the 7B block's flat parameter gathered from 8 ranks
    "llama7b_block_n8_gather": Gather("llama7b_block_n8_gather", LLAMA7B_BLOCK, 8, BF16),
    # the whole 70B flat parameter from 64 ranks' INT8 slots
    "70b_n64_gather": Gather("70b_n64_gather", (70_000_000_000,), 64, BF16),
}


def key_codes(g):
    from .synth import stream_key
    return stream_key("codes", g.name)


def key_scales(g):
    from .synth import stream_key
    return stream_key("scales", g.name)


def key_grad_micro(w, step, micro, k):
    from .synth import stream_key
    return stream_key("grad", w.name, step, "micro", micro, k)


def key_grad(w, step, k):
    from .synth import stream_key
    return stream_key("grad", w.name, step, k)


def key_grad_reduced(w, step):
    from .synth import stream_key
    return stream_key("grad", w.name, step, "reduced")


def key_master(w):
    from .synth import stream_key
    return stream_key("master", w.name)
