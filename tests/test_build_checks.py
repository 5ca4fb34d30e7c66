"""Host-side checks of the build's inline-asm MFMA contract (no GPU): every
asm block that issues an MFMA carries its own wait states, so the compiler
cannot place a read or write of an accumulator inside the MFMA's latency."""
from compressed_sparse_attention_softmax_amd import build

GOOD = """
\t;;#ASMSTART
\ts_nop 1
\tv_mfma_f32_16x16x32_bf16 a[4:7], v[170:173], v[166:169], a[4:7]
\ts_nop 15
\ts_nop 3
\t;;#ASMEND
\tv_accvgpr_mov_b32 a131, a3
"""


def _blocks(text):
    return build.asm_mfma_blocks(text)


def test_self_contained_block_passes():
    b = _blocks(GOOD)
    assert len(b) == 1 and build.asm_mfma_block_ok(b[0])


def test_block_without_tail_fails():
    bad = GOOD.replace("\ts_nop 15\n\ts_nop 3\n", "")
    b = _blocks(bad)
    assert len(b) == 1 and not build.asm_mfma_block_ok(b[0])


def test_short_tail_fails():
    bad = GOOD.replace("\ts_nop 15\n\ts_nop 3\n", "\ts_nop 7\n")
    assert not build.asm_mfma_block_ok(_blocks(bad)[0])


def test_block_without_lead_fails():
    bad = GOOD.replace("\ts_nop 1\n", "", 1)
    assert not build.asm_mfma_block_ok(_blocks(bad)[0])


def test_other_instruction_inside_block_fails():
    bad = GOOD.replace("\ts_nop 15\n", "\tv_accvgpr_read_b32 v1, a4\n\ts_nop 15\n")
    assert not build.asm_mfma_block_ok(_blocks(bad)[0])


def test_blocks_without_mfma_are_ignored():
    assert _blocks("\t;;#ASMSTART\n\ts_nop 15\n\t;;#ASMEND\n") == []
