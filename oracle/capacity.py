"""Block counts and KV byte accounting, as the pages state them.

Test infrastructure only.  Each function restates one formula of the pages
and is pinned in ``tests/test_oracle_pins.py`` to the numbers the pages print
for it (``tests/golden/worked_examples.txt``).
"""


def blocks_needed(n_tokens, block_size):
    """Physical blocks a sequence of ``n_tokens`` occupies: ceil(n / B).

    "vllm-paged-attention-engine" (aiqz.cc), 分页存储设计：标准册页与索引贴纸,
    formula N_i = ceil(S_i / B); "vLLM PagedAttention：大模型推理的显存管理革命"
    (horeb.top), 分配策略 (prefill takes ceil(prompt / 16) blocks).
    """
    if n_tokens < 0 or block_size <= 0:
        raise ValueError("n_tokens >= 0 and block_size > 0 required")
    return -(-n_tokens // block_size)


def last_block_waste(n_tokens, block_size):
    """Empty slots left in a sequence's last block (internal fragmentation).

    "Paged Attention" (daiw.org), 定义 (table: fragmentation is at most the
    last block) and 例子 / 例 2 (worst case B - 1 tokens per sequence).
    """
    return blocks_needed(n_tokens, block_size) * block_size - n_tokens


def worst_case_waste(block_size):
    """Largest possible last-block waste: a sequence one token into a block."""
    return last_block_waste(1, block_size)


def logical_to_physical(block_table, token_index, block_size):
    """(physical block id, slot in block) of logical token ``token_index``.

    "Paged Attention" (daiw.org), 直觉: token i lives in the block that
    block_table[seq][i // block_size] names, at offset i % block_size.
    """
    return block_table[token_index // block_size], token_index % block_size


def kv_bytes(layers, heads, head_dim, seq_len, batch, elem_bytes):
    """KV cache bytes of ``batch`` sequences of ``seq_len`` tokens.

    "vllm-paged-attention-engine" (aiqz.cc), KV缓存之谜, formula
    M_KV = 2 * L * H * d * S * b * P (K and V, every layer, every head).
    """
    return 2 * layers * heads * head_dim * seq_len * batch * elem_bytes


def block_bytes(layers, block_size, kv_heads, head_dim, elem_bytes):
    """Bytes of one physical block across all layers.

    "Paged Attention" (daiw.org), 工程现场：vLLM 块池怎么估容量, step 2:
    2 * L * B * h_kv * d_h * b.
    """
    return 2 * layers * block_size * kv_heads * head_dim * elem_bytes


def pool_blocks(pool_bytes, bytes_per_block):
    """Whole blocks that fit in a pool (same section, step 3)."""
    return pool_bytes // bytes_per_block


def max_concurrency(num_blocks, tokens_per_seq, block_size):
    """Sequences a pool can hold at once (same section, steps 4-5)."""
    return num_blocks // blocks_needed(tokens_per_seq, block_size)
