"""The five workloads (sizes only) and a builder of their seeded device inputs.

  c0  Full-mode decode, batch 1, 4 query tokens, 8,192-token context, m = 1.
  c1  Full-mode decode, batch 32, 131,072 tokens per sequence, m = 2
      (65,536 compressed entries).
  c2  Decoder layer group at 1,048,576 positions (m = 1), batch 8 decode:
      [Full, Reindex, Reuse, Reindex, Reuse, Reindex, Reuse].
  c3  Full-mode prefill chunk: 4,096 query tokens after 262,144 prior tokens,
      m = 2 (133,120 entries visible to the last query).
  c4  Encoder-style group at 1,048,576 tokens, m = 2 (524,288 entries), batch 64
      decode, [Full + 5 Reuse], with the write path and 1% x8 outlier channels.
"""

from dataclasses import dataclass

import torch

from . import (e4m3_rows, head_weights, main_queries, normal_rows, pooled_main_rows,
               token_rows_bf16, outlier_channels)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # layer-group kind: 'full' | 'decoder' | 'encoder'
    B: int
    T: int
    m: int
    n_tokens: int      # tokens before the first query (decode: the context incl. query)
    first_q: int       # token position of the first query of each sequence
    n_cap: int         # compressed entries held per sequence
    outliers: bool = False
    write_path: bool = False

    @property
    def n_layers(self):
        return {"full": 1, "decoder": 7, "encoder": 6}[self.kind]

    @property
    def q_positions(self):
        return [self.first_q + i for i in range(self.T)]

    @property
    def swa_pos0(self):
        return max(0, self.first_q - 127)

    @property
    def S(self):
        return self.first_q + self.T - self.swa_pos0

    def index_layers(self):
        if self.kind == "full":
            return [0]
        if self.kind == "encoder":
            return [0]
        return [0, 1, 3, 5]


WORKLOADS = {
    "c0": Workload("c0", "full", B=1, T=4, m=1, n_tokens=8192, first_q=8188, n_cap=8192),
    "c1": Workload("c1", "full", B=32, T=1, m=2, n_tokens=131072, first_q=131071, n_cap=65536),
    "c2": Workload("c2", "decoder", B=8, T=1, m=1, n_tokens=1048576, first_q=1048575,
                   n_cap=1048576),
    "c3": Workload("c3", "full", B=1, T=4096, m=2, n_tokens=262144 + 4096, first_q=262144,
                   n_cap=133120),
    "c4": Workload("c4", "encoder", B=64, T=1, m=2, n_tokens=1048576, first_q=1048575,
                   n_cap=524288, outliers=True, write_path=True),
}


def scaled(w, n_tokens, n_cap, name=None):
    """A smaller copy of workload `w` with the context cut to `n_tokens` tokens
    held in `n_cap` compressed entries (the queries move to the end)."""
    shift = w.n_tokens - n_tokens
    return Workload(name or (w.name + "_small"), w.kind, w.B, w.T, w.m, n_tokens,
                    w.first_q - shift, n_cap, w.outliers, w.write_path)


def make_inputs(w, device="cuda", seed=0, keep_main_bf16=False, B=None, index_k="fp8"):
    """Device tensors for workload `w` (optionally with fewer sequences B).

    index_k="fp4" draws the indexer keys as bf16 rows of the same N(0,1) draws
    (k_bf16 [B, n_cap, 128]; k_idx is None) for the FP4 indexer-key format; the
    caller quantises them.

    Returns a dict with: k_idx, main_bf16 (only if keep_main_bf16; else None),
    q_idx / w (per index-producing layer), q / swa (per layer), q_pos, swa_pos0,
    and the write-path row (c4)."""
    B = B or w.B
    n_cap, T, L = w.n_cap, w.T, w.n_layers
    out = {"workload": w, "B": B}
    ok = w.outliers
    if index_k == "fp4":
        out["k_idx"] = None
        out["k_bf16"] = normal_rows(B * n_cap, 128, device, seed, w.name, "k_idx",
                                    outliers=ok).to(torch.bfloat16).view(B, n_cap, 128)
    else:
        out["k_idx"] = e4m3_rows(B * n_cap, 128, device, seed, w.name, "k_idx",
                                 outliers=ok).view(B, n_cap, 128)
    main = []
    for b in range(B):
        main.append(pooled_main_rows(n_cap, w.m, device, seed, w.name, "main", b, outliers=ok))
    out["main_bf16"] = torch.stack(main) if keep_main_bf16 else None
    out["main_rows_per_seq"] = main if not keep_main_bf16 else None
    out["q_idx"], out["w"], out["q"], out["swa"] = {}, {}, {}, {}
    for li in w.index_layers():
        out["q_idx"][li] = e4m3_rows(B * T * 32, 128, device, seed, w.name, "q_idx", li,
                                     outliers=ok).view(B, T, 32, 128)
        out["w"][li] = head_weights(B * T, device, seed, w.name, "w", li).view(B, T, 32)
    for li in range(L):
        out["q"][li] = main_queries(B * T, device, seed, w.name, "q", li,
                                    outliers=ok).view(B, T, 64, 512)
        out["swa"][li] = e4m3_rows(B * w.S, 512, device, seed, w.name, "swa", li,
                                   outliers=ok).view(B, w.S, 512)
    qp = torch.tensor(w.q_positions, dtype=torch.int64, device=device)
    out["q_pos"] = qp.view(1, T).expand(B, T).contiguous()
    out["swa_pos0"] = torch.full((B,), w.swa_pos0, dtype=torch.int64, device=device)
    if w.write_path:
        out["write_bf16"] = token_rows_bf16(B, device, seed, w.name, "write", outliers=ok)
    return out


__all__ = ["Workload", "WORKLOADS", "scaled", "make_inputs", "outlier_channels"]
