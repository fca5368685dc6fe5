// gdn_kernels.h -- kernel argument blocks and launchers (host side of the
// kernels; the C ABI in gdn_api.cpp validates arguments and calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct SeqArgs {
    const void* x; int64_t x_stride;
    const void* a; const void* b; int64_t ab_stride;
    int64_t n_rows;
    const int32_t* cu; const int32_t* page_idx; const uint8_t* has_init; int32_t n_seqs;
    const void* conv_w; const float* a_log; const float* dt_bias;
    void* conv_base; int64_t conv_page_stride; int32_t conv_n_pages; uint32_t* sync;
    void* state; int64_t state_page_stride; int32_t state_n_pages;
    float* o;
    int32_t* err;
    int32_t h_k, h_v, d_v;
    float scale, eps;
    // optional: speculative pages whose header each sequence leaves fresh
    uint8_t* spec_pages; int64_t spec_page_bytes; int32_t spec_n_pages;
};

struct ConvArgs {
    const void* x; int64_t x_stride;
    int64_t n_rows;
    const int32_t* cu; const int32_t* page_idx; const uint8_t* has_init; int32_t n_seqs;
    const void* conv_w;
    void* conv_base; int64_t conv_page_stride; int32_t conv_n_pages;
    void* y; int64_t y_stride;
    int32_t* err;
    int32_t C;
    int32_t activation;
};

struct VerifyArgs {
    const void* x; int64_t x_stride;
    const void* a; const void* b; int64_t ab_stride;
    int32_t n_req, n_cand;
    const int32_t* req_page; const int32_t* num_accepted; const uint8_t* step_parity;
    uint8_t* pages; int64_t page_bytes; int32_t n_pages;
    int64_t header_off, state_off, record_off, record_row_bytes;
    const void* conv_w; const float* a_log; const float* dt_bias;
    void* conv_base; int64_t conv_page_stride; int32_t conv_n_pages; uint32_t* sync;
    float* o;
    int32_t* err;
    int32_t h_k, h_v, d_v, n_spec;
    float scale, eps;
    // optional prefix cache: request r writes the committed prefix that ends
    // at replayed record row cache_row[r] into entry cache_entry[r]
    const int32_t* cache_entry; const int32_t* cache_row;
    void* cache_state; int64_t cache_state_stride; int32_t cache_state_n;
    void* cache_conv; int64_t cache_conv_stride; int32_t cache_conv_n;
};

struct RestoreArgs {
    int32_t n_req;
    const int32_t* entry; const int32_t* req_page;
    const void* cache_state; int64_t cache_state_stride; int32_t cache_state_n;
    const void* cache_conv; int64_t cache_conv_stride; int32_t cache_conv_n;
    uint8_t* pages; int64_t page_bytes; int32_t n_pages;
    int64_t header_off, state_off;
    void* conv_base; int64_t conv_page_stride; int32_t conv_n_pages;
    int32_t* err;
    int32_t h_v, d_k, d_v, conv_rows, C;
};

struct ChunkArgs {
    const void* x; int64_t x_stride;
    const void* a; const void* b; int64_t ab_stride;
    int64_t n_rows;
    const int32_t* cu; const int32_t* page_idx; const uint8_t* has_init; int32_t n_seqs;
    const void* conv_w; const float* a_log; const float* dt_bias;
    void* conv_base; int64_t conv_page_stride; int32_t conv_n_pages; uint32_t* sync;
    void* state; int64_t state_page_stride; int32_t state_n_pages;
    float* o;
    int32_t* err;
    int32_t h_k, h_v, d_v;
    float scale, eps;
    void* workspace;  // chunk records (chunked_workspace_bytes), 256-byte aligned
};

// Each returns hipSuccess or the launch error.
hipError_t launch_seq(const SeqArgs& a, int d_k, int act_dtype, int state_dtype, int max_seqlen, hipStream_t s);
hipError_t launch_conv(const ConvArgs& a, int act_dtype, int y_dtype, int max_seqlen, hipStream_t s);
hipError_t launch_verify(const VerifyArgs& a, int d_k, int act_dtype, int state_dtype, int layout,
                         hipStream_t s);
hipError_t launch_restore(const RestoreArgs& a, int act_dtype, int state_dtype, hipStream_t s);
hipError_t launch_chunked(const ChunkArgs& a, int d_k, int act_dtype, int state_dtype, int max_len, hipStream_t s);
size_t chunked_workspace_bytes(int h_k, int h_v, int n_seqs, int64_t n_rows);
// One launch running the token-by-token workgroups of `s` and the verify
// workgroups of `v` (either part may be empty: n_seqs or n_req == 0).
hipError_t launch_mixed(const SeqArgs& s, const VerifyArgs& v, int d_k, int act_dtype, int state_dtype, int layout,
                        hipStream_t st);

// Argument checks and block of a token-by-token call with no caller sync
// words (gdn_api.cpp); GDN_OK with out->n_seqs == 0 for an empty batch.
int32_t seq_call_args_nosync(const struct gdn_dims* dims, const struct gdn_params* params, const void* x,
                             int64_t x_stride, const void* a, const void* b, int64_t ab_stride,
                             const struct gdn_batch* batch, const struct gdn_conv_pool& conv,
                             const struct gdn_state_pool& state, float* o, int32_t* err, SeqArgs* out);

// Which (d_k, d_v) the kernels are compiled for.
bool seq_supported(int d_k, int d_v);
bool chunked_supported(int d_k, int d_v, int chunk);

}  // namespace gdn
