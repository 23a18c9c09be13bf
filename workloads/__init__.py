"""Seeded synthetic inputs for the DSA lightning-indexer + IndexShare + sparse-MLA path.

This module only draws random tensors of the right shapes, dtypes and value
distributions. It holds none of the method's arithmetic: no scoring, no
selection, no attention, no quantisation. Both the CPU oracle's tests and the
HIP path's tests/bench take their inputs from here.

Shapes follow the GLM-5.2 configuration table ("GLM-5.2 总览", table
tbl-glm52-config): a 32-head x 128-dim lightning indexer with top-2048, 64
attention heads, and an MLA latent cache row of 512 latent + 64 RoPE dims in
BF16 (1152 bytes per token per layer).

Every tensor has its own generator, seeded from (seed, tensor tag, layer,
sequence) through splitmix64, so any layer or sequence can be drawn on its own
and large caches are drawn one sequence at a time.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

# ---- model constants (GLM-5.2 总览, tbl-glm52-config; GLM-5.2 架构深度拆解 §1.1) ----
INDEX_HEADS = 32        # index_n_heads
INDEX_DIM = 128         # index_head_dim
TOPK = 2048             # index_topk
MLA_HEADS = 64          # attention heads
LATENT_DIM = 512        # kv_lora_rank
ROPE_DIM = 64           # qk_rope_head_dim
KV_ROW = LATENT_DIM + ROPE_DIM   # 576 bf16 = 1152 B per token per layer
QK_DIM = 256            # qk_nope 192 + qk_rope 64: softmax scale 1/sqrt(256)
N_LAYERS = 78


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: `batch` sequences of `n_ctx` cached tokens, with
    `q_per_seq` query tokens per sequence at the last positions of the context."""
    name: str
    batch: int
    n_ctx: int
    q_per_seq: int
    n_layers: int           # layers the measured unit covers (4 = one F + 3 S group)
    indexer_dtype: str      # "bf16", "fp8", or "fp8h" (fp8 after a Hadamard rotation)
    mla: bool = True        # False: indexer + top-k only (chunked prefill F layer)
    note: str = ""
    kv_dtype: str = "bf16"  # latent cache rows: "bf16" (1152 B) or "fp8" (656 B E4M3 + scales)

    @property
    def n_q(self) -> int:
        return self.batch * self.q_per_seq


WORKLOADS = {
    w.name: w
    for w in [
        Workload("group_b1_n4096_q4", 1, 4096, 4, 4, "bf16",
                 note="tiny IndexShare group, 4 queries at 4092..4095"),
        Workload("decode_b64_n131072", 64, 131072, 1, 4, "bf16",
                 note="decode batch 64 at 128K, one group (1F+3S)"),
        Workload("prefill_q4096_n131072", 1, 131072, 4096, 1, "bf16", mla=False,
                 note="chunked prefill F layer: 4096 queries at 126976..131071"),
        Workload("prefill_q4096_n131072_fp8", 1, 131072, 4096, 1, "fp8", mla=False,
                 note="as above with e4m3 per-128-block indexer q/k"),
        Workload("decode_b8_n1048576_fp8", 8, 1 << 20, 1, 4, "fp8",
                 note="1M-context decode batch 8, fp8 indexer keys, one group"),
        Workload("stack78_b8_q8_n262144", 8, 1 << 18, 8, 78, "bf16",
                 note="78-layer stack (21F+57S), MTP verify shape 8 queries/seq"),
        Workload("prefill_q4096_n131072_fp8h", 1, 131072, 4096, 1, "fp8h", mla=False,
                 note="prefill F layer, Hadamard-rotated e4m3 indexer; the step rotates and quantises q"),
        Workload("decode_b64_n131072_kv8", 64, 131072, 1, 4, "bf16", kv_dtype="fp8",
                 note="decode_b64_n131072 with the FP8 latent cache (656-byte rows)"),
        Workload("decode_b8_n1048576_fp8_kv8", 8, 1 << 20, 1, 4, "fp8", kv_dtype="fp8",
                 note="1M decode with fp8 indexer keys and the FP8 latent cache"),
    ]
}


# ---- seeding ---------------------------------------------------------------
_M64 = (1 << 64) - 1


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _M64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def derive_seed(seed: int, tag: str, *idx: int) -> int:
    h = _splitmix64(seed & _M64)
    for ch in tag.encode():
        h = _splitmix64(h ^ ch)
    for i in idx:
        h = _splitmix64(h ^ (i & _M64))
    return h & ((1 << 63) - 1)


def _gen(device, seed: int, tag: str, *idx: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(derive_seed(seed, tag, *idx))
    return g


def _randint_bf16(shape, lo, hi, g, device):
    return torch.randint(lo, hi + 1, shape, generator=g, device=device,
                         dtype=torch.int32).to(torch.bfloat16)


def _randn_bf16(shape, g, device):
    # fp32 N(0,1) rounded to bf16 (torch's fp32->bf16 cast rounds to nearest even)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


# ---- query layout ----------------------------------------------------------
def query_layout(wl: Workload, device="cpu"):
    """q_seq[i] = sequence of query i; q_pos[i] = its position. Queries of one
    sequence are contiguous and sit at the last q_per_seq positions."""
    i = torch.arange(wl.n_q, dtype=torch.int32)
    q_seq = i // wl.q_per_seq
    q_pos = (wl.n_ctx - wl.q_per_seq) + (i % wl.q_per_seq)
    return q_seq.to(device), q_pos.to(torch.int32).to(device)


# ---- indexer inputs (F layer f) --------------------------------------------
def indexer_keys(wl: Workload, seed: int, f_layer: int, device="cpu", lo=-4, hi=4):
    """k_idx [B, N, 128] bf16, integers uniform in [lo, hi]; one key per position
    shared by all indexer heads."""
    out = torch.empty((wl.batch, wl.n_ctx, INDEX_DIM), dtype=torch.bfloat16, device=device)
    for b in range(wl.batch):
        g = _gen(device, seed, "k_idx", f_layer, b)
        out[b] = _randint_bf16((wl.n_ctx, INDEX_DIM), lo, hi, g, device)
    return out


def indexer_queries(wl: Workload, seed: int, f_layer: int, device="cpu", lo=-4, hi=4):
    """q_idx [n_q, 32, 128] bf16 integers in [lo, hi]; w [n_q, 32] fp32 integers in [1, 4]."""
    g = _gen(device, seed, "q_idx", f_layer)
    q = _randint_bf16((wl.n_q, INDEX_HEADS, INDEX_DIM), lo, hi, g, device)
    g = _gen(device, seed, "w", f_layer)
    w = torch.randint(1, 5, (wl.n_q, INDEX_HEADS), generator=g, device=device,
                      dtype=torch.int32).to(torch.float32)
    return q, w


# ---- MLA inputs (layer l) --------------------------------------------------
def mla_queries(wl: Workload, seed: int, layer: int, device="cpu"):
    """q_lat [n_q, 64, 512] and q_rope [n_q, 64, 64], N(0,1) rounded to bf16;
    drawn separately for every layer."""
    g = _gen(device, seed, "q_lat", layer)
    q_lat = _randn_bf16((wl.n_q, MLA_HEADS, LATENT_DIM), g, device)
    g = _gen(device, seed, "q_rope", layer)
    q_rope = _randn_bf16((wl.n_q, MLA_HEADS, ROPE_DIM), g, device)
    return q_lat, q_rope


def mla_cache(wl: Workload, seed: int, layer: int, device="cpu", seqs=None):
    """kv [B, N, 576] bf16 packed as [512 latent | 64 RoPE key], N(0,1).
    `seqs` draws only those sequences (others are left uninitialised)."""
    out = torch.empty((wl.batch, wl.n_ctx, KV_ROW), dtype=torch.bfloat16, device=device)
    for b in (range(wl.batch) if seqs is None else seqs):
        g = _gen(device, seed, "kv", layer, b)
        out[b] = _randn_bf16((wl.n_ctx, KV_ROW), g, device)
    return out


def mla_cache_seq(wl: Workload, seed: int, layer: int, b: int, device="cpu"):
    """The same rows as mla_cache(...)[b], drawn alone."""
    g = _gen(device, seed, "kv", layer, b)
    return _randn_bf16((wl.n_ctx, KV_ROW), g, device)


def indexer_keys_seq(wl: Workload, seed: int, f_layer: int, b: int, device="cpu", lo=-4, hi=4):
    """The same rows as indexer_keys(...)[b], drawn alone."""
    g = _gen(device, seed, "k_idx", f_layer, b)
    return _randint_bf16((wl.n_ctx, INDEX_DIM), lo, hi, g, device)


# ---- score matrices for stressing the selection alone ------------------------
SCORE_KINDS = ("int_ties", "normal", "all_equal", "signed_zero", "few_values")


def score_matrix(kind: str, n_q: int, n: int, seed: int, device="cpu"):
    """fp32 [n_q, n] score rows for exercising top-k on its own.

    int_ties   : integers ~ round(N(2400, 680)), dense ties like the indexer's
    normal     : N(0, 1) floats
    all_equal  : every score 1.0 (pure tie-break)
    signed_zero: mix of +0.0, -0.0, +-1, +-inf-free negatives
    few_values : only 5 distinct values (huge tie groups)
    """
    g = _gen(device, seed, "scores_" + kind)
    if kind == "int_ties":
        s = torch.randn((n_q, n), generator=g, device=device) * 680.0 + 2400.0
        return torch.round(s).to(torch.float32)
    if kind == "normal":
        return torch.randn((n_q, n), generator=g, device=device, dtype=torch.float32)
    if kind == "all_equal":
        return torch.ones((n_q, n), device=device, dtype=torch.float32)
    if kind == "signed_zero":
        c = torch.randint(0, 4, (n_q, n), generator=g, device=device)
        vals = torch.tensor([0.0, -0.0, 1.0, -1.0], device=device, dtype=torch.float32)
        return vals[c]
    if kind == "few_values":
        c = torch.randint(0, 5, (n_q, n), generator=g, device=device)
        vals = torch.tensor([-2.5, -1.0, 0.0, 3.0, 7.25], device=device, dtype=torch.float32)
        return vals[c]
    raise ValueError(kind)


@dataclass
class GroupInputs:
    """Everything one IndexShare group (1 F layer + n-1 S layers) reads."""
    q_idx: torch.Tensor
    w: torch.Tensor
    k_idx: torch.Tensor
    q_seq: torch.Tensor
    q_pos: torch.Tensor
    layers: list = field(default_factory=list)   # [(q_lat, q_rope, kv), ...]


def group_inputs(wl: Workload, seed: int, f_layer: int = 0, n_layers: int = 4, device="cpu"):
    q_seq, q_pos = query_layout(wl, device)
    q_idx, w = indexer_queries(wl, seed, f_layer, device)
    k_idx = indexer_keys(wl, seed, f_layer, device)
    layers = []
    for l in range(f_layer, f_layer + n_layers):
        q_lat, q_rope = mla_queries(wl, seed, l, device)
        layers.append((q_lat, q_rope, mla_cache(wl, seed, l, device)))
    return GroupInputs(q_idx, w, k_idx, q_seq, q_pos, layers)
