"""Workload shapes: the single linear, the 8B-shaped layer and stacks, the 3B bf16
stack and the 72B-shaped stack that the pages measure or discuss, plus tiny
shapes for tests.  Pure data."""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class ModelCfg:
    name: str
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    n_layers: int
    eps: float
    theta: float
    qkv_bias: bool = False
    tied: bool = False
    quant: str = "nf4"          # "nf4" or "bf16"
    lora_r: int = 16
    lora_alpha: float = 32.0
    batch: int = 1
    seq: int = 512
    n_buffers: int = 2
    loss_chunk: int = 0         # tokens per head / cross-entropy chunk (0 = all)
    wid: int = 0                # seed namespace of the workload

    @property
    def lora_scale(self):
        return self.lora_alpha / self.lora_r

    @property
    def tokens(self):
        return self.batch * self.seq

    def proj_shape(self, name):
        H, I = self.hidden, self.intermediate
        nq, nkv = self.n_heads * self.head_dim, self.n_kv_heads * self.head_dim
        return {"q": (nq, H), "k": (nkv, H), "v": (nkv, H), "o": (H, nq),
                "gate": (I, H), "up": (I, H), "down": (H, I)}[name]

    def with_(self, **kw):
        return replace(self, **kw)


LLAMA8B = dict(hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128, intermediate=14336,
               vocab=128256, eps=1e-5, theta=5e5)
QWEN3B = dict(hidden=2048, n_heads=16, n_kv_heads=2, head_dim=128, intermediate=11008,
              vocab=151936, eps=1e-6, theta=1e6, qkv_bias=True, tied=True)
QWEN72B = dict(hidden=8192, n_heads=64, n_kv_heads=8, head_dim=128, intermediate=29568,
               vocab=152064, eps=1e-6, theta=1e6, qkv_bias=True, tied=False)

# One Llama-3.1-8B-shaped decoder layer, 1 x 2048 tokens.
LAYER_8B = ModelCfg(name="llama8b-layer", n_layers=1, batch=1, seq=2048, wid=2, **LLAMA8B)
# The 32-layer 8B-shaped stack, 1 x 512 tokens, two layer buffers.
STACK_8B = ModelCfg(name="llama8b-stack", n_layers=32, batch=1, seq=512, wid=3, **LLAMA8B)
# Qwen2.5-3B-shaped stack with a bf16 (unquantised) streamed base, 4 x 1024 tokens.
STACK_3B_BF16 = ModelCfg(name="qwen3b-bf16-stack", n_layers=36, batch=4, seq=1024, quant="bf16",
                         wid=4, **QWEN3B)
# Qwen2.5-72B-shaped NF4 stack (layers of ~471 MiB), 1 x 1024 tokens.
STACK_72B = ModelCfg(name="qwen72b-stack", n_layers=80, batch=1, seq=1024, wid=5, **QWEN72B)

# The single NF4 LoRA linear: X [128 x 512], W [1024 x 512], r = 8, alpha = 16.
LINEAR_1 = dict(M=128, K=512, N=1024, r=8, alpha=16.0, wid=1)

# Tiny shapes for CPU and GPU tests (several tiles and a ragged tail on the GPU).
TINY = ModelCfg(name="tiny", hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, intermediate=384,
                vocab=1000, n_layers=3, eps=1e-5, theta=1e4, lora_r=8, lora_alpha=16.0,
                batch=2, seq=80, wid=9)
TINY_QWEN = TINY.with_(name="tiny-qwen", qkv_bias=True, tied=True, quant="bf16", eps=1e-6, wid=10)
