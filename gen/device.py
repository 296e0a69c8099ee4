"""Seeded synthetic linear-draft batches generated on the GPU with torch.

For statistics that need hundreds of batches of the large workload (B=512,
gamma=7, V=128256: 2 GB of bf16 logits per batch), the NumPy builders in
``synth`` are too slow on the host.  This builder draws the same
distributions with torch's seeded device generator instead:

* target logits z_t = s * N(0, 1) in float32 (s = target_std), rounded to
  bf16 (round to nearest even) or kept float32;
* draft logits z_d = z_t + n * N(0, 1) (n = draft_noise), from the rounded
  target, rounded the same way;
* draft tokens: one Gumbel-max draw per drafted row, argmax(z_d / T + G)
  with G = -log(-log(U)), U uniform in (0, 1): an exact draw from
  softmax(z_d / T) of the rounded draft logits, standing in for the drafter;
* uniforms: float32 in [0, 1), [B, gamma + 1].

The values depend only on (seed, shapes, distribution parameters) and the
torch build; they are not the NumPy builder's values.  Like the rest of this
package it holds no verification arithmetic.
"""
import torch


def make_linear_device(B, gamma, V, seed, target_std=2.0, draft_noise=0.8, temperature=0.7, dtype="bf16",
                       device="cuda"):
    """Returns dict(target [B, g+1, V], draft [B, g, V], draft_tokens int32
    [B, g], uniforms float32 [B, g+1], temperature) as device tensors; bf16
    logits come as torch.bfloat16."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    odt = torch.bfloat16 if dtype == "bf16" else torch.float32
    target = (torch.randn((B, gamma + 1, V), generator=gen, device=device) * float(target_std)).to(odt)
    draft = torch.empty((B, gamma, V), dtype=odt, device=device)
    tokens = torch.empty((B, gamma), dtype=torch.int32, device=device)
    for i in range(gamma):                      # one drafted row at a time keeps the float32 temporaries small
        zd = target[:, i].float() + torch.randn((B, V), generator=gen, device=device) * float(draft_noise)
        draft[:, i] = zd.to(odt)
        u = torch.rand((B, V), generator=gen, device=device).clamp_(min=1e-30)
        tokens[:, i] = torch.argmax(draft[:, i].float() / float(temperature) - torch.log(-torch.log(u)),
                                    dim=1).to(torch.int32)
    uniforms = torch.rand((B, gamma + 1), generator=gen, device=device)
    return dict(target=target, draft=draft, draft_tokens=tokens, uniforms=uniforms,
                temperature=float(temperature), dtype=dtype, B=B, gamma=gamma, V=V)
