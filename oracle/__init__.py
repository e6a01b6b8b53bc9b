"""fp64 CPU oracle for fused attention and paged decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's CPU
baseline do.  It shares no code with the HIP library.

What it computes is the plain definition of scaled dot-product attention
("Самовнимание, ядра CUDA и FlashAttention", section 1: the Scores equation
QK^T/sqrt(d_k), the row softmax whose rows sum to one, and the
Attention(Q,K,V) equation; the same explicit softmax(q@k^T/sqrt(d))@v form is
the accuracy check of the "Flash Attention" skill page, scenario 1, step 4).
The fused method reaches this same result up to rounding order (the online
softmax of the same page's section 3 rescales partial outputs "mathematically"),
so the definition itself is the oracle.

Readings where the pages are silent (each listed in the design doc):
  * layout [batch, seq, heads, dim] for q/k/v/out ("Flash Attention" page,
    scenario 2, step 2);
  * GQA/MQA: query head h uses KV head h // (Hq // Hkv) (scenario 2, step 3
    says only that there are fewer KV heads);
  * causal masking is aligned bottom-right: with off = Lk - Lq, query i may
    see key j iff j <= i + off;
  * window = W keeps keys with i + off - W <= j (and j <= i + off + W when
    not causal), the "(left, right)" window of scenario 2, step 3, with
    left = right = W;
  * lse is the natural log of the row's sum of exp(scaled scores), the
    "small normalisation statistics" of section 3 of the self-attention page;
  * a row with no visible key gets out = 0 and lse = -inf;
  * the scale is used as the float32 value a GPU kernel receives;
  * dropout (oracle/dropout.py) drops normalised probabilities, keeps each
    with probability 1 - p, scales the kept ones by 1 / (1 - p), and draws
    its decisions from Philox4x32-10 at a fixed per-element counter.

Parity status of every function here is recorded in tests/test_oracle.py
(all functions are pinned; none is "parity unpinned").
"""
from .core import (  # noqa: F401
    allowed_mask,
    attention_backward,
    kv_head,
    scores,
    attention,
    decode_paged,
    gather_paged_kv,
    online_attention,
    prefill_paged,
    row_softmax,
    split_merge_attention,
)
from .dropout import (  # noqa: F401
    attention_dropout,
    attention_dropout_backward,
    dropout_keep,
    dropout_threshold,
    philox4x32,
)
