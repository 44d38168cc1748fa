"""Synthetic decoder-only transformer for end-to-end training steps with FP8
or bf16 linears (the pages' headline workload: 12 layers, dim 1024, FFN
4096, batch 4 x 512 tokens; [P1] entry reporting the fp8 vs bf16 train step
of that model).  Random weights and random tokens: a timing and
convergence-sanity workload, not a language model.

The qkv, out, up and down projections are the interchangeable linears; the
embedding, norms, attention and the vocabulary head stay in bf16 PyTorch.
Attention runs only on the fused flash / memory-efficient backends."""

from __future__ import annotations

import torch

from .autograd import Fp8Linear


def attention_backends():
    """Context manager restricting scaled_dot_product_attention to the fused
    backends (raises instead of falling back to the math backend)."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    return sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION])


def bf16_linear(i, o, device):
    lin = torch.nn.Linear(i, o, dtype=torch.bfloat16, device=device)
    with torch.no_grad():
        lin.weight.normal_(std=0.02)
        lin.bias.zero_()
    return lin


def fp8_linear(i, o, device):
    return Fp8Linear(i, o, device=device)


class Block(torch.nn.Module):
    def __init__(self, d, heads, ffn, lin, device):
        super().__init__()
        self.h = heads
        self.n1 = torch.nn.RMSNorm(d, dtype=torch.bfloat16, device=device)
        self.n2 = torch.nn.RMSNorm(d, dtype=torch.bfloat16, device=device)
        self.qkv, self.out = lin(d, 3 * d, device), lin(d, d, device)
        self.up, self.down = lin(d, ffn, device), lin(ffn, d, device)

    def forward(self, x):
        B, T, d = x.shape
        q, k, v = self.qkv(self.n1(x)).view(B, T, 3, self.h, d // self.h).permute(2, 0, 3, 1, 4)
        a = torch.nn.functional.scaled_dot_product_attention(
            q.contiguous(), k.contiguous(), v.contiguous(), is_causal=True)
        x = x + self.out(a.transpose(1, 2).reshape(B, T, d))
        return x + self.down(torch.nn.functional.gelu(self.up(self.n2(x))))


class Transformer(torch.nn.Module):
    def __init__(self, lin, layers=12, d=1024, heads=16, ffn=4096, vocab=32000, device="cuda",
                 seed=0):
        super().__init__()
        torch.manual_seed(seed)
        self.emb = torch.nn.Embedding(vocab, d, dtype=torch.bfloat16, device=device)
        self.blocks = torch.nn.ModuleList(Block(d, heads, ffn, lin, device) for _ in range(layers))
        self.norm = torch.nn.RMSNorm(d, dtype=torch.bfloat16, device=device)
        self.head = torch.nn.Linear(d, vocab, bias=False, dtype=torch.bfloat16, device=device)

    def loss(self, tok, tgt):
        x = self.emb(tok)
        for blk in self.blocks:
            x = blk(x)
        logits = self.head(self.norm(x)).float()
        return torch.nn.functional.cross_entropy(logits.view(-1, logits.shape[-1]), tgt.view(-1))


def synthetic_batch(batch, seq, vocab, device, seed=0):
    g = torch.Generator().manual_seed(seed)
    tok = torch.randint(0, vocab, (batch, seq), generator=g)
    tgt = torch.randint(0, vocab, (batch, seq), generator=g)
    return tok.to(device), tgt.to(device)


def train(lin, steps, device, graph=False, warmup=3, seed=0, dims=None, batch=(4, 512)):
    """Train a fresh model (same seed) on one synthetic batch: `warmup`
    eager steps, then `steps` more either eager or as replays of one HIP
    graph holding the whole step (forward, backward, fused AdamW).  Returns
    (losses of the timed steps, ms per timed step)."""
    dims = dims or {}
    vocab = dims.get("vocab", 32000)
    m = Transformer(lin, device=device, seed=seed, **dims)
    tok, tgt = synthetic_batch(batch[0], batch[1], vocab, device, seed=seed)
    opt = torch.optim.AdamW(m.parameters(), lr=1e-4, fused=True, capturable=graph)
    losses = []
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with attention_backends(), torch.cuda.stream(side):
        for _ in range(warmup):
            opt.zero_grad(set_to_none=True)
            m.loss(tok, tgt).backward()
            opt.step()
        if not graph:
            start.record()
            for _ in range(steps):
                opt.zero_grad(set_to_none=True)
                loss = m.loss(tok, tgt)
                loss.backward()
                opt.step()
                losses.append(loss.detach().clone())
            end.record()
        else:
            g = torch.cuda.CUDAGraph()
            opt.zero_grad(set_to_none=True)
            with torch.cuda.graph(g, stream=side):
                loss = m.loss(tok, tgt)
                loss.backward()
                opt.step()
            # the capture ran nothing: replay once per timed step
            start.record()
            for _ in range(steps):
                g.replay()
                losses.append(loss.detach().clone())
            end.record()
    torch.cuda.synchronize()
    return [v.item() for v in losses], start.elapsed_time(end) / steps
