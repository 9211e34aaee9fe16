"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

Holds none of the method's arithmetic: only random draws and tensor shapes.
Every generator takes an explicit seed and device; the same call returns the
same bytes on every run, and both the HIP path and the CPU oracle are fed the
same bytes (the oracle gets a host copy).

Workload recipes (stand-ins for the pages' models; no dataset, no weights):
  * weights / parameters: N(0, 0.02) (0.02 = standard deviation);
  * gradients: N(0, 1e-3), drawn fresh per step from (seed, step);
  * heavy-tailed values: 0.02 * Student-t with 3 degrees of freedom, drawn as
    Z / sqrt(chi2_3 / 3) from four standard normals per value;
  * a 7B decoder's tensors (Llama-2-7B shapes): 32 layers of
    4 x [4096, 4096] (q, k, v, o) and 3 x [4096, 11008] (gate, up, down, the
    last stored as [11008, 4096]), a [32000, 4096] embedding, an untied
    [32000, 4096] output head and 65 RMSNorm vectors of 4096;
  * sparse embedding gradients: a seeded 10% of the 32,000 rows non-zero.
"""
import torch

HIDDEN = 4096
FFN = 11008
VOCAB = 32000
LAYERS = 32


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def normal(n, std, seed, device="cpu", dtype=torch.float32):
    """n values ~ N(0, std^2), drawn in fp32 then cast to dtype (shape [n])."""
    x = torch.empty(int(n), dtype=torch.float32, device=device)
    x.normal_(0.0, std, generator=_gen(seed, device))
    return x if dtype == torch.float32 else x.to(dtype)


def student_t3(n, scale, seed, device="cpu"):
    """n fp32 values ~ scale * Student-t(3)."""
    g = _gen(seed, device)
    z = torch.empty(4, int(n), dtype=torch.float32, device=device).normal_(0.0, 1.0, generator=g)
    chi2 = z[1] * z[1] + z[2] * z[2] + z[3] * z[3]
    return (z[0] / torch.sqrt(chi2 / 3.0)) * scale


def grad_seed(base, tensor_id, step):
    return (int(base) * 1_000_003 + int(tensor_id) * 10_007 + int(step)) & 0x7FFFFFFF


def llama7b_weight_shapes():
    """The 225 weight matrices of a 7B decoder plus its embedding (quantized weights)."""
    shapes = []
    for layer in range(LAYERS):
        for name in ("q", "k", "v", "o"):
            shapes.append((f"layers.{layer}.attn.{name}", (HIDDEN, HIDDEN)))
        shapes.append((f"layers.{layer}.mlp.gate", (FFN, HIDDEN)))
        shapes.append((f"layers.{layer}.mlp.up", (FFN, HIDDEN)))
        shapes.append((f"layers.{layer}.mlp.down", (HIDDEN, FFN)))
    shapes.append(("embed", (VOCAB, HIDDEN)))
    return shapes


def llama7b_param_shapes():
    """The 291 trainable tensors of a 7B decoder: 224 matrices, the embedding,
    an untied output head and 65 RMSNorm vectors (6,738,415,616 parameters)."""
    shapes = [("embed", (VOCAB, HIDDEN))]
    for layer in range(LAYERS):
        shapes.append((f"layers.{layer}.norm_attn", (HIDDEN,)))
        for name in ("q", "k", "v", "o"):
            shapes.append((f"layers.{layer}.attn.{name}", (HIDDEN, HIDDEN)))
        shapes.append((f"layers.{layer}.norm_mlp", (HIDDEN,)))
        shapes.append((f"layers.{layer}.mlp.gate", (FFN, HIDDEN)))
        shapes.append((f"layers.{layer}.mlp.up", (FFN, HIDDEN)))
        shapes.append((f"layers.{layer}.mlp.down", (HIDDEN, FFN)))
    shapes.append(("norm_final", (HIDDEN,)))
    shapes.append(("lm_head", (VOCAB, HIDDEN)))
    return shapes


def sparse_row_grad(rows, cols, frac, std, seed, device="cpu", dtype=torch.bfloat16):
    """[rows, cols] gradient whose rows are zero except a seeded `frac` of them,
    which hold N(0, std^2) values."""
    g = _gen(seed, device)
    k = int(round(rows * frac))
    chosen = torch.randperm(rows, generator=g, device=device)[:k]
    out = torch.zeros(rows, cols, dtype=torch.float32, device=device)
    out[chosen] = torch.empty(k, cols, dtype=torch.float32, device=device).normal_(0.0, std, generator=g)
    return out.to(dtype)
