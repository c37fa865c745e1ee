"""Writes worked_examples.json: hand-derived closed forms of softmax
attention (no library, no oracle, no GPU). Each case carries its derivation.

Run from the repository root:  python tests/golden/make_worked_examples.py
"""
import json
import math
import os

ln = math.log


def cases():
    out = []
    out.append(dict(
        name="two keys with weights 1:3",
        derivation="scores 0 and ln3 give softmax weights 1/4 and 3/4; out = (v0 + 3 v1)/4 = "
                   "([4,-2] + [24,6])/4 = [7,1]; lse = ln(1+3) = ln 4",
        num_q_heads=1, num_kv_heads=1, scale=1.0, context_lens=[2], query_start_loc=None,
        q=[[[1.0, 0.0]]], k=[[[[0.0, 0.0], [ln(3), 5.0]]]], v=[[[[4.0, -2.0], [8.0, 2.0]]]],
        expect_out=[[[7.0, 1.0]]], expect_lse=[[ln(4)]], atol=1e-7))
    out.append(dict(
        name="three keys 1:2:5, GQA 2:1",
        derivation="head 0 (q=[1,0]) scores 0, ln2, ln5 -> weights 1:2:5 of 8: out = "
                   "(v0+2v1+5v2)/8 = ([8,0]+[0,16]+[80,-40])/8 = [11,-3], lse = ln 8; head 1 "
                   "(q=[0,1]) scores all 0 -> mean of v = [8,0], lse = ln 3; both heads read "
                   "the single KV head",
        num_q_heads=2, num_kv_heads=1, scale=1.0, context_lens=[3], query_start_loc=None,
        q=[[[1.0, 0.0], [0.0, 1.0]]], k=[[[[0.0, 0.0], [ln(2), 0.0], [ln(5), 0.0]]]],
        v=[[[[8.0, 0.0], [0.0, 8.0], [16.0, -8.0]]]],
        expect_out=[[[11.0, -3.0], [8.0, 0.0]]], expect_lse=[[ln(8), ln(3)]], atol=1e-6))
    out.append(dict(
        name="causal chunk of 2 at the end of a context of 3",
        derivation="the chunk's tokens sit at positions 1 and 2. Row 0 sees keys 0..1: scores "
                   "0, ln3 -> (4 + 3*8)/4 = 7, lse ln4. Row 1 sees keys 0..2: scores 0, ln3, 0 "
                   "-> (4 + 24 + 100)/5 = 25.6, lse ln5",
        num_q_heads=1, num_kv_heads=1, scale=1.0, context_lens=[3], query_start_loc=[0, 2],
        q=[[[1.0]], [[1.0]]], k=[[[[0.0], [ln(3)], [0.0]]]], v=[[[[4.0], [8.0], [100.0]]]],
        expect_out=[[[7.0]], [[25.6]]], expect_lse=[[ln(4)], [ln(5)]], atol=1e-5))
    L = 17
    out.append(dict(
        name="length-1 sequence and a 17-token sequence crossing a block boundary",
        derivation="seq 0: one key, weight 1: out = v0 = -3, lse = 0.5*2 = 1. seq 1: keys 0..15 "
                   "score 0 (weight 1 each), key 16 scores ln15 (weight 15): Z = 31, out = "
                   "(sum_{t<16} t + 15*16)/31 = 360/31, lse = ln 31",
        num_q_heads=1, num_kv_heads=1, scale=1.0, context_lens=[1, L], query_start_loc=None,
        q=[[[0.5]], [[1.0]]],
        k=[[[[2.0]]], [[[0.0]] * 16 + [[ln(15)]]]],
        v=[[[[-3.0]]], [[[float(t)] for t in range(L)]]],
        expect_out=[[[-3.0]], [[360.0 / 31.0]]], expect_lse=[[1.0], [ln(31)]], atol=1e-5))
    return out


DOC = {
    "source": "Closed forms of softmax attention, derived by hand. The method gathers each "
              "sequence's keys and values through its block table and takes exact softmax "
              "attention over them (page '03 -- Engines Papers', section 2, the PagedAttention "
              "kernel bullet; page 'References', FlashAttention entry: exact attention; a "
              "chunked prefill attends to the K/V already present, first page section 3). The "
              "pages print no worked numeric example; these values follow from the definition "
              "alone.",
}

if __name__ == "__main__":
    DOC["cases"] = cases()
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_examples.json")
    with open(path, "w") as f:
        json.dump(DOC, f, indent=1)
    print("wrote", path)
