// Host-side argument checks for the C ABI in include/lpfa.h. Pure C++: no HIP calls and no
// device reads, so every error path can be exercised without a GPU.
#pragma once
#include <string>

#include "lpfa.h"

namespace lpfa {

// Thread-local message of the last error (lpfa_last_error returns it).
void set_error(const std::string& msg);
void clear_error();
const char* last_error();

// Each returns LPFA_OK or an error code, after recording the message.
int check_quantize(const void* x, int x_dtype, int64_t stride_tok, int64_t stride_head,
                   int64_t total_tokens, int32_t num_heads, int32_t head_dim,
                   const int32_t* cu_seqlens, const int32_t* cu_scale, int32_t num_seqs,
                   int64_t total_scale_rows, int scaling_mode, const uint8_t* payload,
                   const uint8_t* scales);
int check_cast(const void* x, int x_dtype, int64_t stride_tok, int64_t stride_head,
               int64_t total_tokens, int32_t num_heads, int32_t head_dim, const uint8_t* y);
int check_attn(const lpfa_attn_args* a);
int check_bwd(const lpfa_bwd_args* a);

}  // namespace lpfa
