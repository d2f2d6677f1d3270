"""Writes c128_handworked.txt from its closed-form derivation (no oracle, no GPU).

Input (built by handworked.build_handworked): one request, token at position
127 (window rows 0..127, RoPE angle row 0), every state row has
kv_j = +1 if j % 3 == 0 else -1, scores random, RMS weight w_j = 2^(g-3) for
dims j of quant block g = j // 64 < 7 and w_j = 1 on the 64 RoPE dims, eps 0.

Derivation (DeepSeek-V4 fused compress/quant page, sparse-attention kernel):
  pooling: softmax weights sum to 1, so c_j = kv_j = +-1 for every column;
  RMSNorm: mean(c^2) = 1 and eps = 0, so n_j = c_j * w_j = +-2^(g-3);
  bf16 round trip is exact (powers of two);
  block g: absmax A = 2^(g-3); A * fl32(1/448) = 2^(g-3) * fl32(1/448),
    log2 = g - 3 - 8.807..., so e = ceil(.) = g - 11 and the UE8M0 byte is
    e + 127 = 116 + g; the pad byte is 0;
  codes: x = n_j * 2^-e = +-2^(g-3) * 2^(11-g) = +-256 = +-2^8, which is E4M3FN
    0x78 (exponent field 8+7 = 15, mantissa 0), 0xF8 with the sign bit;
  RoPE: angle row 0 holds cos = 1, sin = 0, so the pair is unchanged and
    stored as bf16(+-1) = 0x3F80 / 0xBF80.
"""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def sign(j):
    return 1 if j % 3 == 0 else -1


def main():
    scales = [116 + g for g in range(7)] + [0]
    codes = [0x78 if sign(j) > 0 else 0xF8 for j in range(448)]
    rope = [0x3F80 if sign(448 + k) > 0 else 0xBF80 for k in range(64)]
    lines = [
        "# Hand-derived k_cache record of the input built by handworked.build_handworked().",
        "# Derivation: make_handworked.py (closed form; no oracle or GPU output involved).",
        "# Source of the rules: DeepSeek-V4 fused compress/quant API page (vLLM docs,",
        "# fused_compress_quant_cache), sparse-attention kernel: softmax pooling, RMSNorm,",
        "# UE8M0 exponent ceil(log2(absmax/448)) + 127, E4M3FN codes, GPT-J RoPE, bf16 store.",
        "scales " + " ".join(str(s) for s in scales),
    ]
    for i in range(0, 448, 32):
        lines.append("codes " + " ".join(f"{c:02X}" for c in codes[i:i + 32]))
    for i in range(0, 64, 16):
        lines.append("rope " + " ".join(f"{r:04X}" for r in rope[i:i + 16]))
    with open(os.path.join(HERE, "c128_handworked.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
