"""Parameter, memory, FLOP and byte accounting for the MoE-LoRA layer (host arithmetic only).

Sources:
  [UNS] unsloth.ai "Faster MoE" documentation page (Japanese edition), section
        "Implementation details" and its sub-section on why MoE LoRA differs.
  [ALK] ailinkdeeptech.com cookbook page "Accelerating Mixture-of-Experts Fine-Tuning", section
        "Mathematical Formulation: Split LoRA vs. Standard PEFT".
"""
from __future__ import annotations

__all__ = ["lora_params", "lora_fraction", "peft_delta_elements", "split_memory_crossover",
           "split_memory_crossover_rank", "compute_crossover", "gemm_flops",
           "permute_bytes", "combine_bytes", "combine_bwd_bytes", "unpermute_bytes"]


def lora_params(m: int, n: int, r: int) -> int:
    """Trainable LoRA parameters of one (m, n) projection: m*r + r*n ([UNS] Implementation details)."""
    return m * r + r * n


def lora_fraction(m: int, n: int, r: int) -> float:
    """LoRA parameters as a fraction of the m*n full projection."""
    return lora_params(m, n, r) / (m * n)


def peft_delta_elements(E: int, m: int, n: int) -> int:
    """Elements of the merged delta when materialised for all E experts ([ALK] eq. Memory_PEFT)."""
    return E * m * n


def split_memory_crossover(E: int, m: int, k: int) -> float:
    """[UNS] memory comparison: Split LoRA holds k*s*(r+n) values per projection, the merged path
    E*m*n; with r << n Split LoRA uses less while E*m*n > k*s*n, i.e. s < E*m/k."""
    return E * m / k


def split_memory_crossover_rank(E: int, m: int, n: int, k: int, r: int) -> float:
    """[ALK] section "3. Memory Complexity Crossover": k*s*r < E*m*n  <=>  s < E*m*n/(k*r)."""
    return E * m * n / (k * r)


def compute_crossover(E: int, m: int, n: int, k: int, r: int) -> float:
    """[UNS] FLOP comparison, merged-delta path E(2mnr + mn) + 2k*s*m*n against the split path
    2k(s*m*n + s*m*r + s*r*n): the split path does more work once
    s > E*m*n / (k (m + n)) * (1 + 1/(2r)). (The page prints ~16K for Qwen3-30B-A3B; the formula
    itself gives ~9.0K, and 16K is E*m/(2k), the m = n approximation.)"""
    return E * m * n / (k * (m + n)) * (1.0 + 1.0 / (2.0 * r))


def gemm_flops(s: int, m: int, n: int, E: int, k: int, r: int, backward: bool = True) -> dict:
    """Algorithmic FLOPs of the layer with P = s*k routed pairs.

    forward:  gate_up 2P*m*2n, down 2P*n*m; Split LoRA X A then H_low B per projection:
              gate and up 2 * 2P*r*(m + n), down 2P*r*(n + m)  -> P*(6mn + 6r(m+n)); router 2*s*m*E.
    backward: dX through down 2P*m*n (+ dO B^T, (.)A^T: 2P*r*(m+n)) and gate_up 2P*2n*m
              (+ 4P*r*(m+n)); LoRA-factor gradients X^T(.) and H_low^T(.): 6P*r*(m+n)
              -> P*(6mn + 12 r (m+n)); router 2*s*k*m.
    """
    P = s * k
    fwd_gemm = P * (6 * m * n + 6 * r * (m + n))
    fwd = fwd_gemm + 2 * s * m * E
    out = {"P": P, "fwd": fwd, "fwd_gemm": fwd_gemm, "router_fwd": 2 * s * m * E,
           "gate_up_fwd": 2 * P * m * 2 * n + 4 * P * r * (m + n),
           "down_fwd": 2 * P * n * m + 2 * P * r * (n + m)}
    if backward:
        bwd_gemm = P * (6 * m * n + 12 * r * (m + n))
        out.update(bwd=bwd_gemm + 2 * s * k * m, bwd_gemm=bwd_gemm,
                   gate_up_bwd_dx=2 * P * 2 * n * m + 4 * P * r * (m + n),
                   down_bwd_dx=2 * P * m * n + 2 * P * r * (m + n),
                   lora_grads_bwd=6 * P * r * (m + n))
        out["total"] = out["fwd"] + out["bwd"]
    else:
        out["total"] = out["fwd"]
    return out


def permute_bytes(s: int, m: int, k: int, b: int) -> int:
    """Gather X rows into per-expert order: read s*m*b, write P*m*b, read perm (4P)."""
    P = s * k
    return s * m * b + P * m * b + 4 * P


def combine_bytes(s: int, m: int, k: int, b: int) -> int:
    """Weighted combine: read P*m*b of expert outputs, write s*m*b, read inv and weights (8P)."""
    P = s * k
    return P * m * b + s * m * b + 8 * P


def combine_bwd_bytes(s: int, m: int, k: int, b: int) -> int:
    """dO = w dY and ds = dY.o per row: read dY (s*m*b, once per row through the cache: counted
    once), read o (P*m*b), write dO (P*m*b), perm/weight/ds (12P)."""
    P = s * k
    return s * m * b + 2 * P * m * b + 12 * P


def unpermute_bytes(s: int, m: int, k: int, b: int) -> int:
    """dX[t] = sum_j dXp[inv]: read P*m*b, write s*m*b, read inv (4P)."""
    P = s * k
    return P * m * b + s * m * b + 4 * P
