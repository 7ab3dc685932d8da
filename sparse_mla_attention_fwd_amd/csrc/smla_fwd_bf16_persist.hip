// bf16 KV, 64 heads, one split per token, many tokens: the persistent kernel.
#include "smla_fwd_persist.cuh"
