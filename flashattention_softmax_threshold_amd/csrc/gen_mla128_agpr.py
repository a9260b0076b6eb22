"""Writes mla128_agpr.h: inline-assembly access to the output accumulator of the 128-head MLA
decode kernel (mla128.hip), which keeps O^T in the fixed accumulation registers a0 .. a255.

The assembler takes no register index from a C++ value, so every block of 16 registers gets its
own statement with the register numbers written out; this script writes them. Run it after a
change here (python gen_mla128_agpr.py); the header is committed.
"""
from __future__ import annotations

import os

HERE = os.path.dirname(os.path.abspath(__file__))
NCB = 16  # blocks of 16 registers


def regs(cb: int) -> range:
    return range(16 * cb, 16 * cb + 16)


def asm_lines(instrs: list[str], indent: str) -> list[str]:
    """The asm template as adjacent string literals, one instruction a line."""
    lit = [f'{indent}"{ins}\\n\\t"' for ins in instrs[:-1]] + [f'{indent}"{instrs[-1]}"']
    return lit


def main() -> None:
    out: list[str] = []
    w = out.append
    w("// mla128_agpr.h -- written by gen_mla128_agpr.py; edit that script, not this file.")
    w("//")
    w("// The 128-head MLA decode kernel keeps O^T (16 blocks of 32 x 32 fp32, 256 registers a lane)")
    w("// in the accumulation registers a0 .. a255, block cb in a[16 cb : 16 cb + 15], and touches")
    w("// them only through the statements below. The compiler never sees a value in them: every")
    w("// statement that writes them lists all 256 as clobbered, and the build checks that the")
    w("// compiled kernel uses no accumulation register outside these statements.")
    w("//")
    w("// Wait states the compiler cannot insert for them (it does not look inside the statements):")
    w("// settle() before reading or scaling registers that an MFMA wrote (an 8-pass MFMA result is")
    w("// readable by a vector instruction after at most 11 wait states); a vector write of a")
    w("// register an MFMA reads next needs 2, which scale() and zero_all() end with.")
    w("#pragma once")
    w("")
    w("// Every accumulation register, as an asm clobber list.")
    # wrap the clobber list over several lines
    items = [f'"a{r}"' for r in range(256)]
    w("#define BLASST_AGPR_CLOBBERS \\")
    for i in range(0, 256, 12):
        chunk = ", ".join(items[i:i + 12])
        tail = ", \\" if i + 12 < 256 else ""
        w(f"  {chunk}{tail}")
    w("")
    w("namespace blasst {")
    w("namespace agpr {")
    w("")
    w("typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));")
    w("")
    w("// Wait states after the last MFMA that wrote a block, before a vector read or write of it.")
    w("__device__ __forceinline__ void settle() {")
    w('  asm volatile("s_nop 7\\n\\ts_nop 7\\n\\ts_nop 3");')
    w("}")
    w("")
    w("// a0 .. a255 = 0.")
    w("__device__ __forceinline__ void zero_all() {")
    w("  asm volatile(")
    out.extend(asm_lines([f"v_accvgpr_write_b32 a{r}, 0" for r in range(256)] + ["s_nop 1"],
                         "      "))
    w("      ::: BLASST_AGPR_CLOBBERS);")
    w("}")
    w("")
    w("// Block CB += A B: v_mfma_f32_32x32x16_bf16 with the block as accumulator (C and D).")
    w("template <int CB>")
    w("__device__ __forceinline__ void mfma(const bf16x8_t &a, const bf16x8_t &b);")
    for cb in range(NCB):
        lo, hi = 16 * cb, 16 * cb + 15
        w("template <>")
        w(f"__device__ __forceinline__ void mfma<{cb}>(const bf16x8_t &a, const bf16x8_t &b) {{")
        w(f'  asm volatile("v_mfma_f32_32x32x16_bf16 a[{lo}:{hi}], %0, %1, a[{lo}:{hi}]"')
        w('               :: "v"(a), "v"(b) : BLASST_AGPR_CLOBBERS);')
        w("}")
    w("")
    w("// Block CB *= alpha (alpha: a per-lane value).")
    w("template <int CB>")
    w("__device__ __forceinline__ void scale(float alpha);")
    for cb in range(NCB):
        ins = []
        for r in regs(cb):
            ins += [f"v_accvgpr_read_b32 %0, a{r}", "v_mul_f32 %0, %0, %1",
                    f"v_accvgpr_write_b32 a{r}, %0"]
        w("template <>")
        w(f"__device__ __forceinline__ void scale<{cb}>(float alpha) {{")
        w("  float t;")
        w("  asm volatile(")
        out.extend(asm_lines(ins + ["s_nop 1"], "      "))
        w('      : "=&v"(t) : "v"(alpha) : BLASST_AGPR_CLOBBERS);')
        w("}")
    w("")
    w("// x[i] = register i of block CB.")
    w("template <int CB>")
    w("__device__ __forceinline__ void read(float (&x)[16]);")
    for cb in range(NCB):
        outs = [f'"=v"(x[{i}])' for i in range(16)]
        w("template <>")
        w(f"__device__ __forceinline__ void read<{cb}>(float (&x)[16]) {{")
        w("  asm volatile(")
        out.extend(asm_lines([f"v_accvgpr_read_b32 %{i}, a{r}" for i, r in enumerate(regs(cb))],
                             "      "))
        w("      : " + ", ".join(outs[:8]) + ",")
        w("        " + ", ".join(outs[8:]) + ");")
        w("}")
    w("")
    w("}  // namespace agpr")
    w("}  // namespace blasst")
    with open(os.path.join(HERE, "mla128_agpr.h"), "w") as f:
        f.write("\n".join(out) + "\n")


if __name__ == "__main__":
    main()
