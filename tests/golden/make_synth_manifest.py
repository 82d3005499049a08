"""Write tests/golden/synth_manifest.txt: the SHA-256 of every seeded tensor the
tests and the benchmark draw from bit_quantized_moe_renorm_amd.synth (inputs
only; nothing here computes the block).  Run from the repository root:
    python tests/golden/make_synth_manifest.py
"""
import hashlib
import sys
from pathlib import Path

import numpy as np

sys.path.insert(0, str(Path(__file__).resolve().parents[2]))  # the repository root
from bit_quantized_moe_renorm_amd import synth  # noqa: E402


def tensors():
    """(name, array) for every tensor fingerprinted."""
    out = []
    for tag, spec, seed, fmt in (("tiny_s0", synth.TINY, 0, "q2"), ("ds4_s1", synth.DS4, 1, "q2"),
                                 ("ds4_q4_s1", synth.DS4, 1, "q4")):
        lay = synth.make_layer(spec, seed=seed, fmt=fmt)
        for f in ("router", "router_bias", "gate", "up", "down", "codebook", "sh_gate", "sh_up", "sh_down"):
            a = getattr(lay, f)
            if a is not None:
                out.append((f"{tag}.{f}", a))
    out.append(("hash_table_s1", synth.hash_table(1, synth.N_VOCAB, 256, 6)))
    out.append(("token_ids_s1_1000", synth.token_ids(1, 1000)))
    out.append(("activations_s1_1000x4096_bf16", synth.activations(1, 1000, 4096)))
    out.append(("activations_s0_4x256_f32", synth.activations(0, 4, 256, bf16=False)))
    out.append(("zipf_router_bias_s1", synth.zipf_router_bias(1, 256)))
    out.append(("residual_s41_264x4096", synth.residual(41, 264, 4096)))
    return out


def digest(a):
    a = np.ascontiguousarray(a)
    return hashlib.sha256(str(a.dtype).encode() + str(a.shape).encode() + a.tobytes()).hexdigest()


def main():
    lines = [f"{name} {digest(a)}" for name, a in tensors()]
    (Path(__file__).parent / "synth_manifest.txt").write_text("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
